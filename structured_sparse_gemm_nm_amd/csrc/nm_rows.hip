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

// ---- top-N of a 32-element group by a selection network (M = 32, N = 4 or 8)
//
// Each element gets the unique key (|x| << 6) | ((31 - j) << 1) | sign: larger
// magnitude first, equal magnitudes by lower offset j (the sign never decides,
// since j is unique), and the key still holds the element's bits. Sorting runs
// of four, (for N = 8) merging them into sorted runs of eight, then keeping the
// N largest of each pair of runs (the element-wise maximum of one run against
// the other reversed is the top N, as a bitonic sequence) takes about a third
// of the operations of N rounds of a 32-wide maximum.
__device__ __forceinline__ void cx(uint32_t& a, uint32_t& b) {
  const uint32_t h = max(a, b), l = min(a, b);
  a = h; b = l;
}

template <int L>   // sorts a bitonic run k[o .. o+L) into descending order
__device__ __forceinline__ void bitonic_desc(uint32_t* k) {
#pragma unroll
  for (int st = L / 2; st >= 1; st /= 2)
#pragma unroll
    for (int i = 0; i < L; i++)
      if ((i & st) == 0) cx(k[i], k[i + st]);
}

template <int N>
__device__ __forceinline__ void top_n32(uint32_t (&k)[32], uint32_t (&out)[N]) {
  static_assert(N == 4 || N == 8, "network for N = 4 or 8 of 32");
#pragma unroll
  for (int g = 0; g < 8; g++) {
    cx(k[4 * g], k[4 * g + 1]); cx(k[4 * g + 2], k[4 * g + 3]);
    cx(k[4 * g], k[4 * g + 2]); cx(k[4 * g + 1], k[4 * g + 3]); cx(k[4 * g + 1], k[4 * g + 2]);
  }
  if constexpr (N == 8) {
#pragma unroll
    for (int h = 0; h < 4; h++) {   // runs 2h, 2h+1 -> one sorted run of 8 (second run reversed: bitonic)
      uint32_t t = k[8 * h + 4]; k[8 * h + 4] = k[8 * h + 7]; k[8 * h + 7] = t;
      t = k[8 * h + 5]; k[8 * h + 5] = k[8 * h + 6]; k[8 * h + 6] = t;
      bitonic_desc<8>(k + 8 * h);
    }
  }
#pragma unroll
  for (int runs = 32 / N; runs > 1; runs /= 2) {
#pragma unroll
    for (int i = 0; i < runs / 2; i++) {
      uint32_t c[N];
#pragma unroll
      for (int t = 0; t < N; t++) c[t] = max(k[2 * i * N + t], k[(2 * i + 1) * N + N - 1 - t]);
      if (runs > 2) bitonic_desc<N>(c);
#pragma unroll
      for (int t = 0; t < N; t++) k[i * N + t] = c[t];
    }
  }
#pragma unroll
  for (int t = 0; t < N; t++) out[t] = k[t];
}

template <int DT>
__device__ __forceinline__ uint32_t net_key(uint32_t raw, int j) {
  uint32_t mag, sign;
  if constexpr (DT == DT_I8) {
    const int v = (int)(int8_t)(uint8_t)raw;
    mag = (uint32_t)(v < 0 ? -v : v); sign = v < 0;
  } else {
    mag = raw & 0x7FFFu; sign = raw >> 15;
  }
  return (mag << 6) | ((uint32_t)(31 - j) << 1) | sign;
}

// (offset, bits) of a selected key: rk = (31 - j) << 16 | sign << 15 | magnitude
__device__ __forceinline__ uint32_t by_offset(uint32_t key) {
  return (((key >> 1) & 31u) << 16) | ((key & 1u) << 15) | (key >> 6);
}
template <int DT>
__device__ __forceinline__ uint32_t raw_of(uint32_t rk) {
  if constexpr (DT == DT_I8) {
    const int mag = (int)(rk & 0x7FFFu);
    return (uint32_t)(uint8_t)(((rk >> 15) & 1u) ? -mag : mag);
  } else {
    return rk & 0xFFFFu;
  }
}

enum RowOp { R_PRUNE = 0, R_COMPRESS = 1, R_DECOMPRESS = 2 };

template <int DT, int ESZ, int N, int M, int OP>
__global__ void __launch_bounds__(256) row_kernel(RowArgs A) {
  using G = RowGeom<ESZ, N, M>;
  // decompress at M = 32: one LDS slot per lane (the unit plus 16 bytes, so the
  // 16-byte accesses of 16 consecutive lanes fall on distinct banks)
  // (prune at M = 32 stages its loads and its output the same way, one slot
  // per lane and segment, so that every wave instruction moves 1 KB of
  // contiguous row; a lane reads and then overwrites only its own slot)
  constexpr int SLOT_BYTES = G::UB + 16;
  constexpr bool STAGED = M == 32;
  constexpr bool STAGE_IN = STAGED && OP == R_PRUNE;   // compress reads its units directly (measured faster)
  __shared__ __attribute__((aligned(16))) uint32_t s_unit[STAGED ? G::SPW * 256 * SLOT_BYTES / 4 : 4];
  constexpr int PPU = G::UB / 16;                          // 16-byte pieces per unit
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
    } else if (!STAGE_IN) {
      load_unit<ESZ, G::DW>(d[s], A.a + (r * A.lda + u * G::EPU) * ESZ, vg * G::GD);
    }
  }
  if constexpr (STAGE_IN) {
    // coalesced loads: lane l takes 16-byte piece l % PPU of unit c * 64 / PPU + l / PPU
    u32x4 pc[G::SPW][PPU];
#pragma unroll
    for (int s = 0; s < G::SPW; s++) {
      const int64_t seg = wave * G::SPW + s;
      const int64_t r = seg / A.segs, sr = seg % A.segs;
#pragma unroll
      for (int c = 0; c < PPU; c++) {
        const int uu = c * (64 / PPU) + lane / PPU;
        pc[s][c] = u32x4{0, 0, 0, 0};
        if (r < A.m && sr * 64 + uu < A.units)
          pc[s][c] = __builtin_nontemporal_load(
              (const u32x4*)(A.a + (r * A.lda + (sr * 64 + uu) * G::EPU) * ESZ + 16 * (lane % PPU)));
      }
    }
#pragma unroll
    for (int s = 0; s < G::SPW; s++) {
      uint8_t* wave_slots = (uint8_t*)s_unit + (s * 4 + (threadIdx.x >> 6)) * 64 * SLOT_BYTES;
#pragma unroll
      for (int c = 0; c < PPU; c++)
        *(u32x4*)(wave_slots + (c * (64 / PPU) + lane / PPU) * SLOT_BYTES + 16 * (lane % PPU)) = pc[s][c];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < G::SPW; s++) {
      const uint8_t* mine = (const uint8_t*)s_unit + ((s * 4 + (threadIdx.x >> 6)) * 64 + lane) * SLOT_BYTES;
#pragma unroll
      for (int c = 0; c < PPU; c++) {
        const u32x4 v = *(const u32x4*)(mine + 16 * c);
        d[s][4 * c] = v[0]; d[s][4 * c + 1] = v[1]; d[s][4 * c + 2] = v[2]; d[s][4 * c + 3] = v[3];
      }
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
    if (OP == R_DECOMPRESS && M == 32) {
      // scatter the kept values into the lane's own zeroed LDS slot (in order:
      // later slots win when offsets repeat), then read the unit back
      uint8_t* slot_base = (uint8_t*)s_unit + ((s * 4 + (threadIdx.x >> 6)) * 64 + lane) * SLOT_BYTES;
#pragma unroll
      for (int c = 0; c < G::DW / 4; c++) *(u32x4*)(slot_base + 16 * c) = u32x4{0, 0, 0, 0};
      if (live) {
#pragma unroll
        for (int sl = 0; sl < N; sl++) {
          const int j = (int)((fld[s] >> (sl * G::B)) & (uint64_t)(M - 1));
          const uint32_t v = elem_of<ESZ>(d[s], sl);
          if (ESZ == 2) *(uint16_t*)(slot_base + 2 * j) = (uint16_t)v;
          else slot_base[j] = (uint8_t)v;
        }
      }
      // the wave's 64 units are consecutive in the row: store them as whole
      // 1 KB wave instructions (lane l takes 16-byte piece l % PPU of unit
      // c * 64 / PPU + l / PPU), which keeps every store a full line and lets
      // the dense output stream past the caches
      __syncthreads();
      const uint8_t* wave_slots = (const uint8_t*)s_unit + (s * 4 + (threadIdx.x >> 6)) * 64 * SLOT_BYTES;
#pragma unroll
      for (int c = 0; c < PPU; c++) {
        const int uu = c * (64 / PPU) + lane / PPU;         // unit within the segment
        const u32x4 v = *(const u32x4*)(wave_slots + uu * SLOT_BYTES + 16 * (lane % PPU));
        if (row_ok && sr * 64 + uu < A.units)
          __builtin_nontemporal_store(v, (u32x4*)(A.out + (r * A.lda + (sr * 64 + uu) * G::EPU) * ESZ + 16 * (lane % PPU)));
      }
      continue;
    }
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
    int j2[G::GU][2];                // 2:4: the kept offsets of each group, ascending
    uint32_t sel[N];                 // M = 32: the kept elements as by_offset() keys, offsets ascending
    if constexpr (M == 32) {
      uint32_t key[32];
#pragma unroll
      for (int j = 0; j < 32; j++) key[j] = net_key<DT>(elem_of<ESZ>(d[s], j), j);
      uint32_t top[N];
      top_n32<N>(key, top);
      keep[0] = 0;
#pragma unroll
      for (int t = 0; t < N; t++) {
        sel[t] = by_offset(top[t]);
        keep[0] |= 1u << (31 - (sel[t] >> 16));
      }
      if (OP == R_COMPRESS) {        // offsets ascending = (31 - offset) descending
        if constexpr (N == 4) {
          cx(sel[0], sel[1]); cx(sel[2], sel[3]); cx(sel[0], sel[2]); cx(sel[1], sel[3]); cx(sel[1], sel[2]);
        } else {
          cx(sel[0], sel[1]); cx(sel[2], sel[3]); cx(sel[0], sel[2]); cx(sel[1], sel[3]); cx(sel[1], sel[2]);
          cx(sel[4], sel[5]); cx(sel[6], sel[7]); cx(sel[4], sel[6]); cx(sel[5], sel[7]); cx(sel[5], sel[6]);
          uint32_t t = sel[4]; sel[4] = sel[7]; sel[7] = t;
          t = sel[5]; sel[5] = sel[6]; sel[6] = t;
          bitonic_desc<8>(sel);
        }
      }
      if (vg == 0) keep[0] = 0;
    } else {
#pragma unroll
      for (int g = 0; g < G::GU; g++) {
        uint32_t mag[M];
#pragma unroll
        for (int j = 0; j < M; j++) mag[j] = magkey<DT>(elem_of<ESZ>(d[s], g * M + j));
        if constexpr (M == 4 && N == 2) {
          top2of4(mag, j2[g][0], j2[g][1]);
          keep[g] = g < vg ? (1u << j2[g][0]) | (1u << j2[g][1]) : 0u;
        } else {
          keep[g] = g < vg ? select_topn<M>(mag, N) : 0u;
        }
      }
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
      if constexpr (STAGED) {
        uint8_t* mine = (uint8_t*)s_unit + ((s * 4 + (threadIdx.x >> 6)) * 64 + lane) * SLOT_BYTES;
#pragma unroll
        for (int c = 0; c < PPU; c++)
          *(u32x4*)(mine + 16 * c) = u32x4{d[s][4 * c], d[s][4 * c + 1], d[s][4 * c + 2], d[s][4 * c + 3]};
      } else {
        store_unit<G::DW>(A.out + (r * A.lda + u * G::EPU) * ESZ, d[s], vg * G::GD);
      }
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
    if constexpr (M == 32) {
      if (vg > 0) {
#pragma unroll
        for (int sl = 0; sl < N; sl++) {
          const uint32_t v = raw_of<DT>(sel[sl]);
          const int sft = ESZ == 2 ? 16 * (sl & 1) : 8 * (sl & 3);
          vo[ESZ == 2 ? sl >> 1 : sl >> 2] |= v << sft;
          f |= (uint64_t)(31u - (sel[sl] >> 16)) << (sl * G::B);
        }
      }
    } else if constexpr (M == 4 && N == 2 && ESZ == 2) {
      // the group's elements 0, 1 are dword 2g, elements 2, 3 dword 2g + 1: one
      // byte permute takes elements j0 (low half) and j1 (high half)
#pragma unroll
      for (int g = 0; g < G::GU; g++) {
        if (g >= vg) break;
        const uint32_t jj = (uint32_t)j2[g][0] | ((uint32_t)j2[g][1] << 16);
        vo[g] = __builtin_amdgcn_perm(d[s][2 * g + 1], d[s][2 * g], jj * 0x202u + 0x01000100u);
        f |= (uint64_t)(j2[g][0] | (j2[g][1] << 2)) << (4 * g);
      }
    } else
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
      if constexpr (G::FB == 8 || G::FB == 16) {
        // a unit's field is a whole byte (short): each lane stores its own,
        // contiguous across the wave. The segment's metadata never runs past
        // its 64 units' bytes (the row's padded end is a multiple of 16 bytes
        // and so is every segment start), and lanes past the row's end hold
        // zero fields, which are that padding.
        uint8_t* mp = A.meta + r * A.mld + mbyte0;
        if (lane * (G::FB / 8) < 4 * ndw) {
          if constexpr (G::FB == 8) mp[lane] = (uint8_t)f;
          else *(uint16_t*)(mp + 2 * lane) = (uint16_t)f;
        }
      } else {
        store_seg_meta<G::FB>(A.meta + r * A.mld + mbyte0, f, ndw, lane);
      }
    }
  }
  if constexpr (STAGED && OP == R_PRUNE) {
    // the pruned units went to the lanes' slots: store them as whole 1 KB wave instructions
    __syncthreads();
#pragma unroll
    for (int s = 0; s < G::SPW; s++) {
      const int64_t seg = wave * G::SPW + s;
      const int64_t r = seg / A.segs, sr = seg % A.segs;
      const uint8_t* wave_slots = (const uint8_t*)s_unit + (s * 4 + (threadIdx.x >> 6)) * 64 * SLOT_BYTES;
#pragma unroll
      for (int c = 0; c < PPU; c++) {
        const int uu = c * (64 / PPU) + lane / PPU;
        const u32x4 v = *(const u32x4*)(wave_slots + uu * SLOT_BYTES + 16 * (lane % PPU));
        if (r < A.m && sr * 64 + uu < A.units)
          __builtin_nontemporal_store(v, (u32x4*)(A.out + (r * A.lda + (sr * 64 + uu) * G::EPU) * ESZ + 16 * (lane % PPU)));
      }
    }
  }
}

// ---- prune check for row-contiguous groups: one 16-byte chunk per lane and
// wave instruction (1 KB of row), non-zeros counted per chunk; a group wider
// than 16 bytes spans PPU = M * esize / 16 consecutive lanes, whose counts are
// summed with cross-lane reads (chunks per row is a multiple of PPU, so the
// lanes of a group never straddle a row or a wave).
constexpr int CHECK_CHUNKS_PER_LANE = 4;

template <int DT, int ESZ, int M>
__global__ void __launch_bounds__(256) check_row_kernel(const uint8_t* a, int64_t m, int64_t k, int64_t lda,
                                                        int64_t chunks_row, int N, int32_t* count) {
  constexpr int GB = M * ESZ;
  constexpr int PPU = GB > 16 ? GB / 16 : 1;            // chunks per group
  constexpr int GPC = GB >= 16 ? 1 : 16 / GB;           // groups per chunk
  const int lane = threadIdx.x & 63;
  const int64_t total = m * chunks_row;
  const int64_t nwaves = (total + 64 * CHECK_CHUNKS_PER_LANE - 1) / (64 * CHECK_CHUNKS_PER_LANE);
  const int64_t row_bytes = k * ESZ;
  int bad = 0;
  for (int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); wave < nwaves; wave += (int64_t)gridDim.x * 4) {
  u32x4 v[CHECK_CHUNKS_PER_LANE];
#pragma unroll
  for (int i = 0; i < CHECK_CHUNKS_PER_LANE; i++) {
    const int64_t t = (wave * CHECK_CHUNKS_PER_LANE + i) * 64 + lane;
    v[i] = u32x4{0, 0, 0, 0};
    if (t < total) {
      const int64_t r = t / chunks_row, c = t % chunks_row;
      const uint8_t* p = a + r * lda * ESZ + 16 * c;
      if (16 * c + 16 <= row_bytes) {
        v[i] = *(const u32x4*)p;
      } else {                                          // ragged last chunk: whole groups (dwords) only
        const int nd = (int)((row_bytes - 16 * c) / 4);
#pragma unroll
        for (int d = 0; d < 4; d++) v[i][d] = d < nd ? ((const uint32_t*)p)[d] : 0u;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CHECK_CHUNKS_PER_LANE; i++) {
    const int64_t t = (wave * CHECK_CHUNKS_PER_LANE + i) * 64 + lane;
    int nz[GPC];
#pragma unroll
    for (int g = 0; g < GPC; g++) nz[g] = 0;
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const uint32_t w = v[i][d];
#pragma unroll
      for (int e = 0; e < 4 / ESZ; e++) {
        const uint32_t x = ESZ == 2 ? (w >> (16 * e)) & 0xFFFFu : (w >> (8 * e)) & 0xFFu;
        nz[(d * (4 / ESZ) + e) / (M < 16 / ESZ ? M : 16 / ESZ)] += magkey<DT>(x) != 0u;
      }
    }
    if constexpr (PPU > 1) {
#pragma unroll
      for (int off = 1; off < PPU; off <<= 1) nz[0] += __shfl_xor(nz[0], off);
      if (t < total && lane % PPU == 0) bad += nz[0] > N;
    } else {
#pragma unroll
      for (int g = 0; g < GPC; g++) bad += nz[g] > N;     // zero-filled groups past k count 0
    }
  }
  }
  block_add_count(count, bad);
}

bool check_row_ok(const nm_plan& pl) {
  return pl.p.op_a == NM_OP_N && (pl.p.lda * pl.esz_ab) % 16 == 0;
}

hipError_t launch_check_row(const nm_plan& pl, const void* a, int32_t* count, hipStream_t s) {
  const int64_t chunks_row = (pl.p.k * pl.esz_ab + 15) / 16;
  const int64_t waves = (pl.p.m * chunks_row + 64 * CHECK_CHUNKS_PER_LANE - 1) / (64 * CHECK_CHUNKS_PER_LANE);
  const int64_t blocks = std::min<int64_t>((waves + 3) / 4, kCheckBlocks);
  const uint8_t* ap = (const uint8_t*)a;
  const dim3 grid((unsigned)blocks), block(256);
  const int64_t m = pl.p.m, k = pl.p.k, lda = pl.p.lda;
  const int n = pl.p.nm_n;
#define NM_CHECK_ROW(DT, ESZ, MM) NM_LAUNCH((check_row_kernel<DT, ESZ, MM>), grid, block, 0, s, ap, m, k, lda, chunks_row, n, count)
#define NM_CHECK_ROW_M(DT, ESZ)                         \
  switch (pl.p.nm_m) {                                  \
    case 4: NM_CHECK_ROW(DT, ESZ, 4); break;            \
    case 8: NM_CHECK_ROW(DT, ESZ, 8); break;            \
    case 16: NM_CHECK_ROW(DT, ESZ, 16); break;          \
    default: NM_CHECK_ROW(DT, ESZ, 32); break;          \
  }
  switch (pl.p.type_ab) {
    case NM_F16: NM_CHECK_ROW_M(DT_F16, 2); break;
    case NM_BF16: NM_CHECK_ROW_M(DT_BF16, 2); break;
    default: NM_CHECK_ROW_M(DT_I8, 1); break;
  }
#undef NM_CHECK_ROW_M
#undef NM_CHECK_ROW
  return launch_status();
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

namespace nm {

// ---- 2:4 compress / decompress for groups down stored columns (op_a = T)
//
// Logical row i of op(A) is stored column i, and a group is 4 consecutive
// stored rows of it. A lane takes CPL = LB / esize adjacent stored columns (LB
// bytes of every stored row) over 32 consecutive stored rows (8 groups), so
// each of its 32 loads (stores, for decompress) is LB bytes and a wave
// instruction covers 64 * LB contiguous bytes of a stored row. LB = 8 when
// rows and the base are 8-byte aligned (measured on a 4096 x 11008 operand:
// 16-bit decompress 31 -> 26.5 us, int8 decompress 21 -> 20 us, 16-bit
// compress unchanged), except for int8 compress (29 -> 31 us), which keeps LB =
// 4, as do rows aligned to 4 bytes only. Per logical row
// the 8 groups give 16 kept values (32 bytes for 16-bit types, 16 for int8,
// one or two 16-byte stores) and 32 offset bits (one dword), at offsets that
// are multiples of their size because the 8 groups start at a multiple of 8.
constexpr int CT_GROUPS = 8;                                  // groups per lane
constexpr int CT_ROWS = 4 * CT_GROUPS;                        // stored rows per lane

struct ColTArgs {
  const uint8_t* a;       // stored k x m (compress input)
  uint8_t* out;           // stored k x m (decompress output)
  uint8_t* vals;
  uint8_t* meta;
  int64_t m, k, lda, vld, mld;
  int64_t col_lanes;      // lanes across the stored columns: ceil(m / CPL)
};

template <int DT, int ESZ, int OP, int LB>
__global__ void __launch_bounds__(256) colT24_kernel(ColTArgs A) {
  constexpr int CPL = LB / ESZ;                               // stored columns per lane
  constexpr int NW = LB / 4;                                  // dwords per lane and stored row
  constexpr int VBYTES = CT_GROUPS * 2 * ESZ;                 // kept-value bytes per logical row and lane
  // a block's four waves take four consecutive 32-row blocks of the same 64
  // column lanes (64 CPL logical rows, 128 stored rows)
  const int64_t ncg = (A.col_lanes + 63) / 64;
  const int64_t cg = blockIdx.x % ncg, kg = blockIdx.x / ncg;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t cl = cg * 64 + lane, kb = kg * 4 + wv;        // column lane, 32-row block
  const int64_t c0 = cl * CPL, s0 = kb * CT_ROWS;             // first stored column, first stored row
  // 16-bit types, every lane of the block with whole columns and 8 whole
  // groups: the kept values and offsets go through LDS so that each global
  // store (compress) or load (decompress) instruction covers whole 128-byte
  // pieces of 8 compressed rows (a lane owns logical rows, so its own
  // accesses would touch 64 rows each)
  constexpr int LR = 64 * CPL;                                // logical rows per block
  constexpr int VP = 4 * VBYTES + 16;                         // LDS pitch of a logical row's values (padded)
  constexpr int CH = 4 * VBYTES / 16;                         // 16-byte chunks of a logical row in the block
  const bool staged = ESZ == 2 && (kg * 4 + 4) * CT_ROWS <= A.k && (cg + 1) * LR <= A.m;
  const int64_t i0 = cg * LR;                                 // the block's first logical row
  const int64_t vbb = (kg * 4 * CT_ROWS / 4) * 2 * ESZ;      // its first value byte in a row (2 kept per group)
  const int64_t mbb = kg * 4 * CT_ROWS / 8;                   // its first offset byte in a row
  if (s0 >= A.k) return;
  const int groups_here = (int)min((int64_t)CT_GROUPS, (A.k - s0) / 4);
  const int cols_here = (int)min((int64_t)CPL, A.m - c0);
  if (cols_here <= 0) return;
  const bool full_cols = cols_here == CPL;
  const bool last_kb = s0 + CT_ROWS >= A.k;
  auto elem = [&](const uint32_t (&w)[NW], int c) -> uint32_t {
    return (w[(c * ESZ) / 4] >> (8 * ((c * ESZ) % 4))) & (ESZ == 2 ? 0xFFFFu : 0xFFu);
  };
  if constexpr (OP == R_COMPRESS) {
    __shared__ __attribute__((aligned(16))) uint8_t s_vals[ESZ == 2 ? LR * VP : 16];
    __shared__ __attribute__((aligned(16))) uint32_t s_meta[ESZ == 2 ? LR * 4 : 4];
    uint32_t w[CT_ROWS][NW];
#pragma unroll
    for (int r = 0; r < CT_ROWS; r++) {
#pragma unroll
      for (int d = 0; d < NW; d++) w[r][d] = 0;
      if (r < 4 * groups_here) {
        const uint8_t* p = A.a + ((s0 + r) * A.lda + c0) * ESZ;
        if (full_cols) {
          if constexpr (NW == 2) {
            const u32x2 v = *(const u32x2*)p;
            w[r][0] = v[0]; w[r][1] = v[1];
          } else {
            w[r][0] = *(const uint32_t*)p;
          }
        } else {
#pragma unroll
          for (int c = 0; c < CPL; c++)                       // unrolled: the word index stays static
            if (c < cols_here)
              w[r][(c * ESZ) / 4] |= (ESZ == 2 ? (uint32_t)((const uint16_t*)p)[c] : (uint32_t)p[c]) << (8 * ((c * ESZ) % 4));
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      if (c >= cols_here) break;
      const int64_t i = c0 + c;                               // logical row
      uint32_t vo[VBYTES / 4];
#pragma unroll
      for (int x = 0; x < VBYTES / 4; x++) vo[x] = 0;
      uint32_t mw = 0;
#pragma unroll
      for (int g = 0; g < CT_GROUPS; g++) {
        if (g >= groups_here) break;
        uint32_t mag[4], raw[4];
#pragma unroll
        for (int j = 0; j < 4; j++) { raw[j] = elem(w[4 * g + j], c); mag[j] = magkey<DT>(raw[j]); }
        int j0, j1;
        top2of4(mag, j0, j1);
        const uint32_t v0 = j0 == 0 ? raw[0] : j0 == 1 ? raw[1] : j0 == 2 ? raw[2] : raw[3];
        const uint32_t v1 = j1 == 0 ? raw[0] : j1 == 1 ? raw[1] : j1 == 2 ? raw[2] : raw[3];
        const int s = 2 * g;                                  // first slot of the group
        if (ESZ == 2) { vo[g] = v0 | (v1 << 16); }
        else { vo[s >> 2] |= (v0 << (8 * (s & 3))) | (v1 << (8 * ((s + 1) & 3))); }
        mw |= (uint32_t)(j0 | (j1 << 2)) << (4 * g);
      }
      uint8_t* vrow = A.vals + i * A.vld * ESZ;
      const int64_t vb0 = (s0 / 4) * 2 * ESZ;                 // byte offset of this lane's first value
      uint8_t* mrow = A.meta + i * A.mld;
      const int64_t mb0 = s0 / 8;                             // 4 bits per group
      if (staged) {
        const int lr = lane * CPL + c;                        // logical row in the block
#pragma unroll
        for (int x = 0; x < VBYTES / 16; x++)
          *(u32x4*)(s_vals + lr * VP + wv * VBYTES + 16 * x) = u32x4{vo[4 * x], vo[4 * x + 1], vo[4 * x + 2], vo[4 * x + 3]};
        s_meta[lr * 4 + wv] = mw;
      } else if (groups_here == CT_GROUPS) {
#pragma unroll
        for (int x = 0; x < VBYTES / 16; x++)
          *(u32x4*)(vrow + vb0 + 16 * x) = u32x4{vo[4 * x], vo[4 * x + 1], vo[4 * x + 2], vo[4 * x + 3]};
      } else {
        const int nb = groups_here * 2 * ESZ;                 // value bytes present (even)
        for (int x = 0; x < nb / 4; x++) *(uint32_t*)(vrow + vb0 + 4 * x) = vo[x];
        if (nb & 2) *(uint16_t*)(vrow + vb0 + 4 * (nb / 4)) = (uint16_t)vo[nb / 4];
      }
      if (!staged) {
        if (groups_here == CT_GROUPS) *(uint32_t*)(mrow + mb0) = mw;
        else for (int x = 0; x < groups_here / 2 + (groups_here & 1); x++) mrow[mb0 + x] = (uint8_t)(mw >> (8 * x));
      }
      if (last_kb) {                                          // zero padding of both compressed rows
        const int64_t vend = vb0 + groups_here * 2 * ESZ;
        for (int64_t b = vend; b < A.vld * ESZ; b++) vrow[b] = 0;
        const int64_t mend = mb0 + (groups_here + 1) / 2;
        for (int64_t b = mend; b < A.mld; b++) mrow[b] = 0;
      }
    }
    if (staged) {                                             // uniform over the block (depends on its index only)
      __syncthreads();
#pragma unroll
      for (int j = 0; j < LR * CH / 256; j++) {
        const int q = threadIdx.x + 256 * j;
        const int row = q / CH, ch = q % CH;
        *(u32x4*)(A.vals + (i0 + row) * A.vld * ESZ + vbb + 16 * ch) = *(const u32x4*)(s_vals + row * VP + 16 * ch);
      }
#pragma unroll
      for (int j = 0; j < LR * 4 / 256; j++) {
        const int q = threadIdx.x + 256 * j;
        *(uint32_t*)(A.meta + (i0 + q / 4) * A.mld + mbb + 4 * (q % 4)) = s_meta[q];
      }
    }
  } else {  // decompress
    __shared__ __attribute__((aligned(16))) uint8_t s_vals[ESZ == 2 ? LR * VP : 16];
    __shared__ __attribute__((aligned(16))) uint32_t s_meta[ESZ == 2 ? LR * 4 : 4];
    if (staged) {                                             // uniform over the block (depends on its index only)
#pragma unroll
      for (int j = 0; j < LR * CH / 256; j++) {
        const int q = threadIdx.x + 256 * j;
        const int row = q / CH, ch = q % CH;
        *(u32x4*)(s_vals + row * VP + 16 * ch) = *(const u32x4*)(A.vals + (i0 + row) * A.vld * ESZ + vbb + 16 * ch);
      }
#pragma unroll
      for (int j = 0; j < LR * 4 / 256; j++) {
        const int q = threadIdx.x + 256 * j;
        s_meta[q] = *(const uint32_t*)(A.meta + (i0 + q / 4) * A.mld + mbb + 4 * (q % 4));
      }
      __syncthreads();
    }
    uint32_t w[CT_ROWS][NW];
#pragma unroll
    for (int r = 0; r < CT_ROWS; r++)
#pragma unroll
      for (int d = 0; d < NW; d++) w[r][d] = 0;
#pragma unroll
    for (int c = 0; c < CPL; c++) {
      if (c >= cols_here) continue;                           // (not break: the loop stays fully unrolled)
      const int64_t i = c0 + c;
      const uint8_t* vrow = A.vals + i * A.vld * ESZ;
      const int64_t vb0 = (s0 / 4) * 2 * ESZ;
      uint32_t vo[VBYTES / 4];
      uint32_t mw = 0;
      if (staged) {
        const int lr = lane * CPL + c;                        // logical row in the block
#pragma unroll
        for (int x = 0; x < VBYTES / 16; x++) {
          const u32x4 v = *(const u32x4*)(s_vals + lr * VP + wv * VBYTES + 16 * x);
          vo[4 * x] = v[0]; vo[4 * x + 1] = v[1]; vo[4 * x + 2] = v[2]; vo[4 * x + 3] = v[3];
        }
        mw = s_meta[lr * 4 + wv];
      } else {
        if (groups_here == CT_GROUPS) {
#pragma unroll
          for (int x = 0; x < VBYTES / 16; x++) {
            const u32x4 v = *(const u32x4*)(vrow + vb0 + 16 * x);
            vo[4 * x] = v[0]; vo[4 * x + 1] = v[1]; vo[4 * x + 2] = v[2]; vo[4 * x + 3] = v[3];
          }
        } else {
          const int nb = groups_here * 2 * ESZ;               // value bytes present (even)
#pragma unroll
          for (int x = 0; x < VBYTES / 4; x++) vo[x] = x < nb / 4 ? *(const uint32_t*)(vrow + vb0 + 4 * x) : 0u;
          if (nb & 2) vo[nb / 4] = *(const uint16_t*)(vrow + vb0 + 4 * (nb / 4));
        }
        const uint8_t* mrow = A.meta + i * A.mld;
        const int64_t mb0 = s0 / 8;
        if (groups_here == CT_GROUPS) mw = *(const uint32_t*)(mrow + mb0);
        else for (int x = 0; x < (groups_here + 1) / 2; x++) mw |= (uint32_t)mrow[mb0 + x] << (8 * x);
      }
#pragma unroll
      for (int g = 0; g < CT_GROUPS; g++) {
        if (g >= groups_here) break;
#pragma unroll
        for (int sl = 0; sl < 2; sl++) {                      // later slot wins on a repeated offset
          const int j = (int)((mw >> (4 * g + 2 * sl)) & 3u);
          const int s = 2 * g + sl;
          const uint32_t v = ESZ == 2 ? (vo[s >> 1] >> (16 * (s & 1))) & 0xFFFFu : (vo[s >> 2] >> (8 * (s & 3))) & 0xFFu;
          const int d = (ESZ * c) / 4;
          const uint32_t sh = 8 * ((ESZ * c) % 4);
          const uint32_t msk = (ESZ == 2 ? 0xFFFFu : 0xFFu) << sh;
#pragma unroll
          for (int jj = 0; jj < 4; jj++)
            if (j == jj) w[4 * g + jj][d] = (w[4 * g + jj][d] & ~msk) | (v << sh);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < CT_ROWS; r++) {
      if (r >= 4 * groups_here) continue;                     // (not break: the loop stays fully unrolled)
      uint8_t* p = A.out + ((s0 + r) * A.lda + c0) * ESZ;
      if (full_cols) {
        if constexpr (NW == 2) *(u32x2*)p = u32x2{w[r][0], w[r][1]};
        else *(uint32_t*)p = w[r][0];
      } else {
#pragma unroll
        for (int c = 0; c < CPL; c++) {                       // unrolled: the word index stays static
          if (c >= cols_here) break;
          const uint32_t v = w[r][(c * ESZ) / 4] >> (8 * ((c * ESZ) % 4));
          if (ESZ == 2) ((uint16_t*)p)[c] = (uint16_t)v;
          else p[c] = (uint8_t)v;
        }
      }
    }
  }
}

bool colT_path_ok(const nm_plan& pl) {
  return pl.p.op_a == NM_OP_T && pl.p.nm_n == 2 && pl.p.nm_m == 4 && (pl.p.lda * pl.esz_ab) % 4 == 0;
}

template <int OP, int LB>
static hipError_t launch_colT_lb(const nm_plan& pl, ColTArgs A, hipStream_t s) {
  const int cpl = LB / pl.esz_ab;
  A.m = pl.p.m; A.k = pl.p.k; A.lda = pl.p.lda; A.vld = pl.vld; A.mld = pl.mld;
  A.col_lanes = (A.m + cpl - 1) / cpl;
  const int64_t row_blocks = (A.k + CT_ROWS - 1) / CT_ROWS;
  const int64_t blocks = ((A.col_lanes + 63) / 64) * ((row_blocks + 3) / 4);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (pl.p.type_ab) {
    case NM_F16: NM_LAUNCH((colT24_kernel<DT_F16, 2, OP, LB>), dim3((unsigned)blocks), dim3(256), 0, s, A); break;
    case NM_BF16: NM_LAUNCH((colT24_kernel<DT_BF16, 2, OP, LB>), dim3((unsigned)blocks), dim3(256), 0, s, A); break;
    default:
      if constexpr (OP == R_COMPRESS && LB == 8) return hipErrorInvalidValue;   // not used (see above)
      else NM_LAUNCH((colT24_kernel<DT_I8, 1, OP, LB>), dim3((unsigned)blocks), dim3(256), 0, s, A);
      break;
  }
  return launch_status();
}

// 8 bytes per lane and stored row when every row start is 8-byte aligned
// (int8 compress: 4)
template <int OP>
static hipError_t launch_colT(const nm_plan& pl, ColTArgs A, const void* dense, hipStream_t s) {
  const bool wide = (pl.p.lda * pl.esz_ab) % 8 == 0 && (uintptr_t)dense % 8 == 0;
  if (wide && (pl.esz_ab == 2 || OP == R_DECOMPRESS)) return launch_colT_lb<OP, 8>(pl, A, s);
  return launch_colT_lb<OP, 4>(pl, A, s);
}

hipError_t launch_colT_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s) {
  ColTArgs A{};
  A.a = (const uint8_t*)a; A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta;
  return launch_colT<R_COMPRESS>(pl, A, a, s);
}

hipError_t launch_colT_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s) {
  ColTArgs A{};
  A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta; A.out = (uint8_t*)out;
  return launch_colT<R_DECOMPRESS>(pl, A, out, s);
}

}  // namespace nm
