// Internal declarations shared by the nmsparse host code and kernels (not
// installed, not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/nmsparse.h"

struct nm_plan {
  nm_problem_t p;
  int esz_ab;           // bytes per A/B element
  int esz_cd;           // bytes per C/D element
  int64_t a_rows;       // stored A rows  (m for op N, k for op T)
  int64_t a_cols;       // stored A cols  (k for op N, m for op T)
  int bits;             // metadata bits per kept element: ceil(log2 M)
  int vrows;            // rows of op(A) sharing one kept-offset set (1: element-wise N:M; >1: vector-wise)
  int vshift;           // log2(vrows): metadata row of op(A) row r is r >> vshift
  int64_t vld;          // values row stride (elements)
  int64_t mld;          // metadata row stride (bytes)
  int kernel;           // SpMM kernel id (nm::KernelId)
  std::string spmm_symbol;  // device kernel nm_spmm launches (filled on first query)
  int force_tile;           // -1 = automatic, else nm::TileCfg (set through the algorithm id)
  int algorithm;            // nm_plan_set_algorithm id (NM_ALG_AUTO unless set)
  int split_k;              // nm_plan_set_split_k: requested k ranges of the 2:4 product (1 = none)
  bool tile_elemwise;       // NM_TILE_ELEMWISE (read once at plan creation): prune/check/compress/decompress
                            // on the LDS tile kernels even where the register path applies
};

namespace nm {

// block tile of the matrix-core kernels
enum TileCfg { T128 = 0, T256x128 = 1, T256 = 2 };

enum KernelId {
  K_NONE = 0,
  K_SMFMAC_24 = 1,      // 2:4 on the sparse matrix instructions
  K_GATHER_MFMA = 2,    // general N:M: A expanded in registers, dense MFMA
  K_SKINNY = 3,         // small n: streamed A, B in LDS, VALU gather
  K_VW_MFMA = 4,        // vector-wise N:M: B rows gathered per 16-row block, dense MFMA on the kept k
};

void set_error(const std::string& msg);

// Dry run of a launch: while the calling thread's probe is armed, NM_LAUNCH
// records the kernel's host stub instead of launching it, so the same host
// logic that picks a kernel can also name it.
// The first kernel recorded is the product's main kernel (a split-k product
// launches its reduction afterwards).
struct LaunchProbe {
  bool armed = false;
  const void* kernel = nullptr;
};
LaunchProbe& launch_probe();
inline hipError_t launch_status() { return launch_probe().armed ? hipSuccess : hipGetLastError(); }
#define NM_LAUNCH(KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                              \
  do {                                                                                  \
    if (::nm::launch_probe().armed) {                                                   \
      if (!::nm::launch_probe().kernel) ::nm::launch_probe().kernel = (const void*)(KERNEL); \
    } else {                                                                            \
      hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);              \
    }                                                                                   \
  } while (0)

// Split-k of the 2:4 product: the k ranges nm_spmm launches for this plan (1
// when the plan asks for none or its shape does not take the whole-tile
// copy-ring kernel), and the workspace bytes they need: one m x n plane of
// fp32 / int32 partial sums per range.
int spmm_splits(const nm_plan& pl);
size_t spmm_workspace_bytes(const nm_plan& pl);
constexpr int MAX_SPLIT_K = 16;

// ---- launchers (return hipError_t from the launch) ----
hipError_t launch_prune_1d(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
// register path for op_a = N with 16-byte rows and N:M in {2:4, 4:32, 8:32}
bool row_path_ok(const nm_plan& pl);
hipError_t launch_row_prune(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
hipError_t launch_row_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s);
hipError_t launch_row_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s);
// 2:4 compress / decompress for op_a = T (groups down stored columns), dword-aligned stored rows
bool colT_path_ok(const nm_plan& pl);
hipError_t launch_colT_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s);
hipError_t launch_colT_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s);
// 1-D prune check for op_a = N with 16-byte rows, any N:M (the counter must already be zero)
bool check_row_ok(const nm_plan& pl);
hipError_t launch_check_row(const nm_plan& pl, const void* a, int32_t* count, hipStream_t s);
hipError_t launch_prune_tile(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
hipError_t launch_mask_apply(const nm_plan& pl, const uint32_t* mask, void* x, hipStream_t s);
hipError_t launch_check(const nm_plan& pl, const void* a, int mode, int32_t* count, hipStream_t s);
hipError_t launch_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s);
hipError_t launch_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s);
hipError_t launch_spmm_smfmac(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, void* ws, hipStream_t s);
// vector-wise N:M (vrows > 1, op_a = N): prune, check, compress, decompress
hipError_t launch_vw_prune(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
hipError_t launch_vw_check(const nm_plan& pl, const void* a, int32_t* count, hipStream_t s);
hipError_t launch_vw_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s);
hipError_t launch_vw_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s);
// whether the vector-wise matrix-core product takes this plan (whole tiles, B stored k x n, ...)
bool vw_mfma_ok(const nm_plan& pl);
hipError_t launch_spmm_vw(const nm_plan& pl, float alpha, const void* vals, const void* meta, const void* b,
                          float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_spmm_gather(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_spmm_skinny(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_dense_gemm(const nm_plan& pl, float alpha, const void* a, const void* b, float beta,
                             const void* c, void* d, hipStream_t s);

}  // namespace nm
