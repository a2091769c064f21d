// Vector-wise N:M: prune, prune check, compress and decompress (HBM-bound).
//
// What they compute (apex PR "[sparse] update support for arbitrary N:M
// settings sparse", extension 2, vector-wise N:M for nmSPARSE): the V
// consecutive rows of a block of op(A) share one set of kept offsets per group
// of M columns. A vector is the block's V values in one column, scored by the
// absolute value of their sum (the signed values added first, in fp64, in row
// order), and the N best-scoring vectors of every group are kept for all V
// rows, ties to the lower offset. Scores compare as the bit patterns of the
// non-negative fp64 values (NaN above +Inf). Values keep the element-wise
// compressed layout; the metadata has one bit-stream row per block.
//
// Design: a block of 256 threads owns one V-row block x 256 columns; thread t
// owns column c0 + t of all V rows, so every row access of a wave is 128
// (16-bit) or 64 (int8) contiguous bytes. A group of M columns lies in M
// consecutive lanes of one wave; each lane ranks its score against the other
// M - 1 of its group with cross-lane reads. A chunk of 256 columns holds a
// whole number of metadata bytes for every N:M, so a block assembles its
// chunk's bits in LDS and writes them as whole bytes; the block holding a
// row's last chunk also writes the zero padding of the values and metadata.
#include "nm_internal.h"
#include "nm_device.h"

namespace nm {

constexpr int VW_COLS = 256;   // columns (threads) per block

struct VwArgs {
  const uint8_t* a;      // stored op(A) (m x k, lda) for prune / check / compress
  uint8_t* out;          // pruned or decompressed op(A) (lda)
  uint32_t* mask;        // optional keep mask (prune)
  uint8_t* vals;         // compressed values (vld elements per row)
  uint8_t* meta;         // metadata, one row of mld bytes per block of V rows
  int32_t* count;        // check: non-conforming (block, group) pairs
  int64_t m, k, lda, vld, mld, mask_ld;
  int V, N, M, bits;
};

enum VwOp { VW_PRUNE = 0, VW_CHECK = 1, VW_COMPRESS = 2, VW_DECOMPRESS = 3 };

template <int ESZ>
__device__ __forceinline__ uint32_t ld_raw(const uint8_t* p, int64_t idx) {
  return ESZ == 2 ? (uint32_t)((const uint16_t*)p)[idx] : (uint32_t)p[idx];
}
template <int ESZ>
__device__ __forceinline__ void st_raw(uint8_t* p, int64_t idx, uint32_t v) {
  if (ESZ == 2) ((uint16_t*)p)[idx] = (uint16_t)v;
  else p[idx] = (uint8_t)v;
}

// The element's value in fp64 (exact for every fp16, bf16 and int8 value).
template <int DT>
__device__ __forceinline__ double val64(uint32_t raw) {
  if constexpr (DT == DT_F16) return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)raw);
  else if constexpr (DT == DT_BF16) return (double)__builtin_bit_cast(float, raw << 16);
  else return (double)(int)(int8_t)(uint8_t)raw;
}

template <int DT>
__device__ __forceinline__ bool nonzero(uint32_t raw) {
  if constexpr (DT == DT_I8) return (raw & 0xFFu) != 0u;
  else return (raw & 0x7FFFu) != 0u;     // -0 counts as zero
}

template <int DT, int OP>
__global__ void __launch_bounds__(VW_COLS) vw_elem_kernel(VwArgs A) {
  constexpr int ESZ = DT == DT_I8 ? 1 : 2;
  __shared__ uint32_t s_bits[80];      // the chunk's metadata bits (at most 8 groups x 31 x 5 = 1240 bits)
  const int t = threadIdx.x, lane = t & 63;
  const int64_t blk = blockIdx.y;
  const int64_t r0 = blk * A.V;
  const int64_t c0 = (int64_t)blockIdx.x * VW_COLS;
  const int64_t c = c0 + t;
  const bool in = c < A.k;                               // k % M == 0: a group is wholly in or out
  const int M = A.M, N = A.N, b = A.bits;
  const int j = lane & (M - 1);                          // offset in the group (M divides 64)
  const int gl = t / M;                                  // group within the chunk
  const int64_t g = c / M;                               // group within the row
  const int64_t chunk_groups = ((A.k - c0 < VW_COLS ? A.k - c0 : VW_COLS)) / M;
  const uint64_t group_lanes = (M == 64 ? ~0ull : ((1ull << M) - 1ull)) << (lane - j);
  const bool last_chunk = c0 + VW_COLS >= A.k;
  // metadata bits of this chunk start on a byte boundary (256 / M * N * b is a multiple of 8)
  const int64_t byte0 = (c0 / M) * N * b / 8;
  const int nbytes = (int)((chunk_groups * N * b + 7) / 8);

  if constexpr (OP == VW_CHECK) {
    // the grid strides down the row blocks
    int bad = 0;
    for (int64_t rb = blk; rb < A.m / A.V; rb += gridDim.y) {
      bool nz = false;
      for (int v = 0; v < A.V; v++) nz |= in && nonzero<DT>(ld_raw<ESZ>(A.a, (rb * A.V + v) * A.lda + c));
      const uint64_t used = __ballot(nz) & group_lanes;
      bad += (j == 0 && in && __popcll(used) > N) ? 1 : 0;
    }
    block_add_count(A.count, bad);
    return;
  }

  if constexpr (OP == VW_DECOMPRESS) {
    // the chunk's metadata bytes into LDS, then each lane finds its offset among its group's N fields
    uint8_t* sb = (uint8_t*)s_bits;
    for (int x = t; x < (int)sizeof(s_bits); x += VW_COLS) sb[x] = 0;
    __syncthreads();
    for (int x = t; x < nbytes; x += VW_COLS) sb[x] = A.meta[blk * A.mld + byte0 + x];
    __syncthreads();
    int slot = -1;
    if (in) {
      for (int s = 0; s < N; s++) {
        const int p = (gl * N + s) * b;
        const uint32_t w = (uint32_t)sb[p / 8] | ((uint32_t)sb[p / 8 + 1] << 8);
        if ((int)((w >> (p % 8)) & (uint32_t)(M - 1)) == j) slot = s;
      }
    }
    for (int v = 0; v < A.V; v++) {
      const int64_t r = r0 + v;
      if (!in) continue;
      const uint32_t val = slot >= 0 ? ld_raw<ESZ>(A.vals, r * A.vld + g * N + slot) : 0u;
      st_raw<ESZ>(A.out, r * A.lda + c, val);
    }
    return;
  }

  // ---- prune / compress: the vector score and the rank inside the group ----
  double sum = 0.0;
  for (int v = 0; v < A.V; v++) sum += in ? val64<DT>(ld_raw<ESZ>(A.a, (r0 + v) * A.lda + c)) : 0.0;
  const uint64_t key = __builtin_bit_cast(uint64_t, sum) & 0x7FFFFFFFFFFFFFFFull;   // bits of |sum|
  const uint32_t klo = (uint32_t)key, khi = (uint32_t)(key >> 32);
  int rank = 0;
  for (int i = 0; i < M; i++) {
    const int src = lane - j + i;
    const uint32_t olo = __shfl(klo, src), ohi = __shfl(khi, src);
    const uint64_t other = ((uint64_t)ohi << 32) | olo;
    rank += (other > key || (other == key && i < j)) ? 1 : 0;
  }
  const bool keep = in && rank < N;
  const uint64_t kept = __ballot(keep);

  if constexpr (OP == VW_PRUNE) {
    for (int v = 0; v < A.V; v++) {
      const int64_t r = r0 + v;
      if (in) st_raw<ESZ>(A.out, r * A.lda + c, keep ? ld_raw<ESZ>(A.a, r * A.lda + c) : 0u);
    }
    if (A.mask) {
      // the wave's 64 columns are two mask words of every row of the block
      const int64_t cw = c0 + (t & ~63);
      if (cw < A.k) {
        const int64_t w0 = cw / 32;
        for (int v = lane; v < A.V; v += 64) {
          A.mask[(r0 + v) * A.mask_ld + w0] = (uint32_t)kept;
          if (cw + 32 < A.k) A.mask[(r0 + v) * A.mask_ld + w0 + 1] = (uint32_t)(kept >> 32);
        }
      }
    }
    return;
  }

  // ---- compress: values to their slots, offsets into the chunk's bit image ----
  const int slot = __popcll(kept & group_lanes & ((1ull << lane) - 1ull));
  for (int x = t; x < 80; x += VW_COLS) s_bits[x] = 0u;
  __syncthreads();
  if (keep) {
    for (int v = 0; v < A.V; v++) {
      const int64_t r = r0 + v;
      st_raw<ESZ>(A.vals, r * A.vld + g * N + slot, ld_raw<ESZ>(A.a, r * A.lda + c));
    }
    const int p = (gl * N + slot) * b;
    atomicOr(&s_bits[p / 32], (uint32_t)j << (p % 32));
    if (p % 32 + b > 32) atomicOr(&s_bits[p / 32 + 1], (uint32_t)j >> (32 - p % 32));
  }
  __syncthreads();
  const uint8_t* sb = (const uint8_t*)s_bits;
  for (int x = t; x < nbytes; x += VW_COLS) A.meta[blk * A.mld + byte0 + x] = sb[x];
  if (last_chunk) {
    // zero padding: metadata bytes after the stream, values after k N / M
    for (int64_t x = byte0 + nbytes + t; x < A.mld; x += VW_COLS) A.meta[blk * A.mld + x] = 0;
    const int64_t kv = A.k / M * N;
    for (int v = 0; v < A.V; v++)
      for (int64_t x = kv + t; x < A.vld; x += VW_COLS) st_raw<ESZ>(A.vals, (r0 + v) * A.vld + x, 0u);
  }
}

static VwArgs make_vw_args(const nm_plan& pl) {
  VwArgs A{};
  A.m = pl.p.m; A.k = pl.p.k; A.lda = pl.p.lda; A.vld = pl.vld; A.mld = pl.mld;
  A.mask_ld = (pl.p.k + 31) / 32;
  A.V = pl.vrows; A.N = pl.p.nm_n; A.M = pl.p.nm_m; A.bits = pl.bits;
  return A;
}

template <int OP>
static hipError_t launch_vw(const nm_plan& pl, const VwArgs& A, hipStream_t s) {
  if (A.m == 0 || A.k == 0) return hipSuccess;
  const int64_t gx = (A.k + VW_COLS - 1) / VW_COLS, gy = A.m / A.V;
  const dim3 grid((unsigned)gx, (unsigned)(OP == VW_CHECK ? std::min<int64_t>(gy, std::max<int64_t>(1, kCheckBlocks / gx)) : gy));
  switch (pl.p.type_ab) {
    case NM_F16: hipLaunchKernelGGL((vw_elem_kernel<DT_F16, OP>), grid, dim3(VW_COLS), 0, s, A); break;
    case NM_BF16: hipLaunchKernelGGL((vw_elem_kernel<DT_BF16, OP>), grid, dim3(VW_COLS), 0, s, A); break;
    default: hipLaunchKernelGGL((vw_elem_kernel<DT_I8, OP>), grid, dim3(VW_COLS), 0, s, A); break;
  }
  return hipGetLastError();
}

__global__ void vw_zero_kernel(int32_t* p) { *p = 0; }

hipError_t launch_vw_prune(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s) {
  VwArgs A = make_vw_args(pl);
  A.a = (const uint8_t*)a; A.out = (uint8_t*)out; A.mask = mask;
  return launch_vw<VW_PRUNE>(pl, A, s);
}

hipError_t launch_vw_check(const nm_plan& pl, const void* a, int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(vw_zero_kernel, dim3(1), dim3(1), 0, s, count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  VwArgs A = make_vw_args(pl);
  A.a = (const uint8_t*)a; A.count = count;
  return launch_vw<VW_CHECK>(pl, A, s);
}

hipError_t launch_vw_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s) {
  VwArgs A = make_vw_args(pl);
  A.a = (const uint8_t*)a; A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta;
  return launch_vw<VW_COMPRESS>(pl, A, s);
}

hipError_t launch_vw_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s) {
  VwArgs A = make_vw_args(pl);
  A.vals = (uint8_t*)vals; A.meta = (uint8_t*)meta; A.out = (uint8_t*)out;
  return launch_vw<VW_DECOMPRESS>(pl, A, s);
}

}  // namespace nm
