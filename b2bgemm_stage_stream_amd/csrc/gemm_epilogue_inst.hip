// One instantiation unit of the GEMM + epilogue kernel, compiled once per
// (input dtype, B layout, part) so that the units build in parallel:
// CF_IN_F32 in {0, 1}, CF_B_NK in {0, 1}, and CF_PART
//   0 to 4    fast path, row op CF_PART (with and without bias/residual);
//   5 to 9    general (element-masked) path, row op CF_PART - 5;
//   10 to 18  two row stages, fast path: first row op 1 + (CF_PART - 10) / 3,
//             second 1 + (CF_PART - 10) % 3 (bf16 inputs only);
//   19        top-k with lists of 8, fast path (bf16 inputs only);
//   20        top-k with lists of 4 (k <= 4), fast path (bf16 inputs only);
//   21 to 23  column reductions (softmax, LayerNorm, RMSNorm over the rows
//             of each column), fast path.
#include "gemm_epilogue_kernel.hpp"

#if !defined(CF_IN_F32) || !defined(CF_B_NK) || !defined(CF_PART)
#error "CF_IN_F32, CF_B_NK and CF_PART must be defined"
#endif
#if CF_IN_F32 && CF_PART >= 10 && CF_PART <= 20
#error "two-stage and top-k parts are built for bf16 inputs only"
#endif

#define CF_JOIN2(a, b) a##b
#define CF_JOIN(a, b) CF_JOIN2(a, b)
#define CF_FN CF_JOIN(cf_ge_kernels_, CF_JOIN(CF_IN_F32, CF_JOIN(_, CF_JOIN(CF_B_NK, CF_JOIN(_, CF_PART)))))

namespace cf {

// Kernel entry of this unit; `pre` selects the bias/residual variant (the
// general path always takes the bias/residual code).
const void* CF_FN(int pre) {
  constexpr bool kF = CF_IN_F32 != 0, kN = CF_B_NK != 0;
#if CF_PART < 5
  if (pre) return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART, true>;
  return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART, false>;
#elif CF_PART < 10
  (void)pre;
  return (const void*)&gemm_epilogue_kernel<kF, kN, false, CF_PART - 5, true>;
#elif CF_PART < 19
  if (pre) return (const void*)&gemm_epilogue_kernel<kF, kN, true, 1 + (CF_PART - 10) / 3, true, 1 + (CF_PART - 10) % 3>;
  return (const void*)&gemm_epilogue_kernel<kF, kN, true, 1 + (CF_PART - 10) / 3, false, 1 + (CF_PART - 10) % 3>;
#elif CF_PART < 21
  // epilogue ROW 5: lists of 8; ROW 6: lists of 4
  if (pre) return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART - 14, true>;
  return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART - 14, false>;
#else
  // epilogue ROW 7, 8, 9: column softmax, LayerNorm, RMSNorm
  if (pre) return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART - 14, true>;
  return (const void*)&gemm_epilogue_kernel<kF, kN, true, CF_PART - 14, false>;
#endif
}

}  // namespace cf
