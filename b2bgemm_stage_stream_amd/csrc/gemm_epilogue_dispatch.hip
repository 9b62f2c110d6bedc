// Host-side selection and launch of the GEMM + epilogue kernel instantiations,
// and the workspace clear kernel.
#include "cf_launch.h"

#include <mutex>

namespace cf {

// The occupancy query and the device attribute read cost microseconds of host
// time, which small launches would pay on every call; both are fixed per
// (device, kernel), so they are cached. A full table leaves new entries
// uncached (still correct).
namespace {
struct OccEntry {
  const void* k;
  int dev, threads, n;
};
std::mutex g_occ_mu;
OccEntry g_occ[512];
int g_occ_used = 0;
int g_cus[64];   // 0: not read yet
}  // namespace

hipError_t blocks_per_cu_cached(const void* k, int threads, int* n) {
  *n = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> g(g_occ_mu);
    for (int i = 0; i < g_occ_used; ++i)
      if (g_occ[i].k == k && g_occ[i].dev == dev && g_occ[i].threads == threads) {
        *n = g_occ[i].n;
        return hipSuccess;
      }
  }
  int v = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, k, threads, 0)) != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_occ_mu);
  if (g_occ_used < (int)(sizeof(g_occ) / sizeof(g_occ[0]))) g_occ[g_occ_used++] = OccEntry{k, dev, threads, v};
  *n = v;
  return hipSuccess;
}

hipError_t device_cus_cached(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> g(g_occ_mu);
    if (g_cus[dev] > 0) {
      *cus = g_cus[dev];
      return hipSuccess;
    }
  }
  int v = 0;
  if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> g(g_occ_mu);
    g_cus[dev] = v;
  }
  *cus = v;
  return hipSuccess;
}

// Instantiation units (gemm_epilogue_inst.hip): parts 0-9 for both input
// dtypes, parts 10-20 (two row stages, top-k) for bf16 inputs only.
#define CF_DECL10(F, N)                                                                              \
  const void* cf_ge_kernels_##F##_##N##_0(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_1(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_2(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_3(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_4(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_5(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_6(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_7(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_8(int);                                                      \
  const void* cf_ge_kernels_##F##_##N##_9(int);
#define CF_DECL_BF16_EXTRA(N)                                                                        \
  const void* cf_ge_kernels_0_##N##_10(int);                                                         \
  const void* cf_ge_kernels_0_##N##_11(int);                                                         \
  const void* cf_ge_kernels_0_##N##_12(int);                                                         \
  const void* cf_ge_kernels_0_##N##_13(int);                                                         \
  const void* cf_ge_kernels_0_##N##_14(int);                                                         \
  const void* cf_ge_kernels_0_##N##_15(int);                                                         \
  const void* cf_ge_kernels_0_##N##_16(int);                                                         \
  const void* cf_ge_kernels_0_##N##_17(int);                                                         \
  const void* cf_ge_kernels_0_##N##_18(int);                                                         \
  const void* cf_ge_kernels_0_##N##_19(int);                                                         \
  const void* cf_ge_kernels_0_##N##_20(int);
#define CF_DECL_COL(F, N)                                                                            \
  const void* cf_ge_kernels_##F##_##N##_21(int);                                                     \
  const void* cf_ge_kernels_##F##_##N##_22(int);                                                     \
  const void* cf_ge_kernels_##F##_##N##_23(int);
CF_DECL10(0, 0)
CF_DECL10(0, 1)
CF_DECL10(1, 0)
CF_DECL10(1, 1)
CF_DECL_BF16_EXTRA(0)
CF_DECL_BF16_EXTRA(1)
CF_DECL_COL(0, 0)
CF_DECL_COL(0, 1)
CF_DECL_COL(1, 0)
CF_DECL_COL(1, 1)

typedef const void* (*PartFn)(int);
constexpr int kNumParts = 24;
#define CF_ROW10(F, N)                                                                               \
  cf_ge_kernels_##F##_##N##_0, cf_ge_kernels_##F##_##N##_1, cf_ge_kernels_##F##_##N##_2,             \
      cf_ge_kernels_##F##_##N##_3, cf_ge_kernels_##F##_##N##_4, cf_ge_kernels_##F##_##N##_5,         \
      cf_ge_kernels_##F##_##N##_6, cf_ge_kernels_##F##_##N##_7, cf_ge_kernels_##F##_##N##_8,         \
      cf_ge_kernels_##F##_##N##_9
#define CF_ROW_EXTRA(N)                                                                              \
  cf_ge_kernels_0_##N##_10, cf_ge_kernels_0_##N##_11, cf_ge_kernels_0_##N##_12,                      \
      cf_ge_kernels_0_##N##_13, cf_ge_kernels_0_##N##_14, cf_ge_kernels_0_##N##_15,                  \
      cf_ge_kernels_0_##N##_16, cf_ge_kernels_0_##N##_17, cf_ge_kernels_0_##N##_18,                  \
      cf_ge_kernels_0_##N##_19, cf_ge_kernels_0_##N##_20
#define CF_ROW_COL(F, N) cf_ge_kernels_##F##_##N##_21, cf_ge_kernels_##F##_##N##_22, cf_ge_kernels_##F##_##N##_23
#define CF_NULL11 nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr
static const PartFn kParts[2][2][kNumParts] = {
    {{CF_ROW10(0, 0), CF_ROW_EXTRA(0), CF_ROW_COL(0, 0)}, {CF_ROW10(0, 1), CF_ROW_EXTRA(1), CF_ROW_COL(0, 1)}},
    // fp32 inputs: parts 10-20 absent (null)
    {{CF_ROW10(1, 0), CF_NULL11, CF_ROW_COL(1, 0)}, {CF_ROW10(1, 1), CF_NULL11, CF_ROW_COL(1, 1)}}};

static const void* part(bool in_f32, bool b_nk, int i, int pre) {
  const PartFn f = kParts[in_f32][b_nk][i];
  return f ? f(pre) : nullptr;
}

// Null when no instantiation serves the combination (the C ABI refuses those
// before it gets here).
static const void* pick(const GemmEpilogueParams& p, bool in_f32, bool b_nk, bool vec) {
  // two row stages: fast path only, one part per (first, second) row op
  if (p.row_op2 != 0) {
    const bool ok = vec && p.row_op >= 1 && p.row_op <= 3 && p.row_op2 >= 1 && p.row_op2 <= 3;
    return ok ? part(in_f32, b_nk, 10 + 3 * (p.row_op - 1) + (p.row_op2 - 1),
                     (p.bias != nullptr || p.residual != nullptr) ? 1 : 0)
              : nullptr;
  }
  if (p.col) {   // column reductions: fast path, parts 21-23 for softmax, LayerNorm, RMSNorm
    const bool ok = vec && p.row_op >= 1 && p.row_op <= 3;
    return ok ? part(in_f32, b_nk, 20 + p.row_op, (p.bias != nullptr || p.residual != nullptr) ? 1 : 0) : nullptr;
  }
  if (p.row_op == 5)   // top-k: lists of 4 when k <= 4, else of 8
    return vec ? part(in_f32, b_nk, p.topk <= 4 ? 20 : 19, (p.bias != nullptr) ? 1 : 0) : nullptr;
  if (p.row_op < 0 || p.row_op > 4) return nullptr;
  return part(in_f32, b_nk, vec ? p.row_op : 5 + p.row_op, (p.bias != nullptr || p.residual != nullptr) ? 1 : 0);
}

int gemm_epilogue_blocks_per_cu(const GemmEpilogueParams& p, bool in_f32, bool b_nk, bool vec) {
  const void* k = pick(p, in_f32, b_nk, vec);
  int n = 0;
  if (k == nullptr || blocks_per_cu_cached(k, 256, &n) != hipSuccess) return 0;
  return n;
}

hipError_t launch_gemm_epilogue(const GemmEpilogueParams& p, bool in_f32, bool b_nk, bool vec, int grid,
                                hipStream_t stream) {
  const void* k = pick(p, in_f32, b_nk, vec);
  if (k == nullptr) return hipErrorInvalidDeviceFunction;
  void* args[] = {(void*)&p};
  return hipLaunchKernel(k, dim3(grid), dim3(256), args, 0, stream);
}

// Clears a workspace with a fill kernel (no hipMemsetAsync, so the call can be
// captured in a graph).
__global__ void workspace_clear_kernel(uint32_t* ws, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    ws[i] = 0u;
}

hipError_t launch_workspace_clear(void* ws, size_t bytes, hipStream_t stream) {
  const size_t words = bytes / 4;
  const size_t want = (words + 255) / 256;
  const int blocks = (int)(want < 1024 ? want : 1024);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(workspace_clear_kernel, dim3(blocks), dim3(256), 0, stream, (uint32_t*)ws, words);
  return hipGetLastError();
}

}  // namespace cf
