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
  int64_t vld;          // values row stride (elements)
  int64_t mld;          // metadata row stride (bytes)
  int kernel;           // SpMM kernel id (nm::KernelId)
};

namespace nm {

enum KernelId {
  K_NONE = 0,
  K_SMFMAC_24 = 1,      // 2:4 on the sparse matrix instructions
  K_GATHER_MFMA = 2,    // general N:M: A expanded in registers, dense MFMA
  K_SKINNY = 3,         // small n: streamed A, B in LDS, VALU gather
};

void set_error(const std::string& msg);

// ---- launchers (return hipError_t from the launch) ----
hipError_t launch_prune_1d(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
hipError_t launch_prune_tile(const nm_plan& pl, const void* a, void* out, uint32_t* mask, hipStream_t s);
hipError_t launch_check(const nm_plan& pl, const void* a, int mode, int32_t* count, hipStream_t s);
hipError_t launch_compress(const nm_plan& pl, const void* a, void* vals, void* meta, hipStream_t s);
hipError_t launch_decompress(const nm_plan& pl, const void* vals, const void* meta, void* out, hipStream_t s);
hipError_t launch_spmm_smfmac(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_spmm_gather(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_spmm_skinny(const nm_plan& pl, float alpha, const void* vals, const void* meta,
                              const void* b, float beta, const void* c, void* d, hipStream_t s);
hipError_t launch_dense_gemm(const nm_plan& pl, float alpha, const void* a, const void* b, float beta,
                             const void* c, void* d, hipStream_t s);

}  // namespace nm
