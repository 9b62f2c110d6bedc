// One instantiation unit of the GEMM + epilogue kernel. Compiled once per
// (input dtype, B layout, part): CF_IN_F32 in {0, 1}, CF_B_NK in {0, 1},
// CF_PART in {0, 1, 2, 3, 4} (fast path for row op CF_PART, with and without
// bias/residual), 5 (general path), 6 to 14 (two row stages, fast path:
// first row op 1 + (CF_PART - 6) / 3, second 1 + (CF_PART - 6) % 3), 15 (top-k, fast path) or 16 (top-k with
// k <= 4, fast path).
// Splitting the instantiations lets them compile in parallel.
#include "gemm_epilogue_kernel.hpp"

#if !defined(CF_IN_F32) || !defined(CF_B_NK) || !defined(CF_PART)
#error "CF_IN_F32, CF_B_NK and CF_PART must be defined"
#endif

#define CF_JOIN2(a, b) a##b
#define CF_JOIN(a, b) CF_JOIN2(a, b)
#define CF_FN CF_JOIN(cf_ge_kernels_, CF_JOIN(CF_IN_F32, CF_JOIN(_, CF_JOIN(CF_B_NK, CF_JOIN(_, CF_PART)))))

namespace cf {

// Kernel entry of this unit; `pre` selects the bias/residual variant (every
// part but the general one).
const void* CF_FN(int pre) {
#if CF_PART < 5
  if (pre) return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, CF_PART, true>;
  return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, CF_PART, false>;
#elif CF_PART == 5
  (void)pre;
  return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, false, 0, false>;
#elif CF_PART == 15 || CF_PART == 16
  if (pre) return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, CF_PART - 10, true>;
  return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, CF_PART - 10, false>;
#else
  if (pre)
    return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, 1 + (CF_PART - 6) / 3, true,
                                              1 + (CF_PART - 6) % 3>;
  return (const void*)&gemm_epilogue_kernel<CF_IN_F32 != 0, CF_B_NK != 0, true, 1 + (CF_PART - 6) / 3, false,
                                            1 + (CF_PART - 6) % 3>;
#endif
}

}  // namespace cf
