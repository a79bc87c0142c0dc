// LDS-layout variants of the 256 x 256 fp16 -> fp16 GEMM (kernel in gemm_pp_kernel.hpp).
//
// The operand swizzles are members of the chunk-XOR family of "CUDA Swizzle & bank conflict"
// (section "Triton - Shared Layout swizzling": vec, perPhase, maxPhase), on 16-byte chunks. Each
// variant computes the same values as the default kernel (the layout only decides where an operand
// chunk sits in LDS, never the arithmetic); what changes is how many LDS bank conflicts the operand
// reads incur. The set compiled here spans no swizzle, partial swizzles and the default for each
// operand, with the other operand at its default.
#include "gemm_pp_kernel.hpp"

namespace tbl {
namespace {

struct LayoutVariant {
  int a_pp, a_mp, b_vec, b_pp, b_mp;
  hipError_t (*launch)(const GemmLaunch&, hipStream_t);
};

constexpr LayoutVariant kVariants[] = {
    {4, 4, 4, 1, 4, &launch_pp_typed<false, false, 4, 4, 4, 1, 4>},   // the default layouts
    {1, 1, 4, 1, 4, &launch_pp_typed<false, false, 1, 1, 4, 1, 4>},   // A unswizzled
    {1, 4, 4, 1, 4, &launch_pp_typed<false, false, 1, 4, 4, 1, 4>},
    {2, 4, 4, 1, 4, &launch_pp_typed<false, false, 2, 4, 4, 1, 4>},
    {4, 2, 4, 1, 4, &launch_pp_typed<false, false, 4, 2, 4, 1, 4>},
    {8, 4, 4, 1, 4, &launch_pp_typed<false, false, 8, 4, 4, 1, 4>},
    {4, 4, 1, 1, 1, &launch_pp_typed<false, false, 4, 4, 1, 1, 1>},   // B unswizzled
    {4, 4, 1, 1, 4, &launch_pp_typed<false, false, 4, 4, 1, 1, 4>},
    {4, 4, 2, 1, 4, &launch_pp_typed<false, false, 4, 4, 2, 1, 4>},
    {4, 4, 4, 1, 2, &launch_pp_typed<false, false, 4, 4, 4, 1, 2>},
    {4, 4, 4, 2, 2, &launch_pp_typed<false, false, 4, 4, 4, 2, 2>},
    {4, 4, 8, 1, 4, &launch_pp_typed<false, false, 4, 4, 8, 1, 4>},
};

const LayoutVariant* find(int a_pp, int a_mp, int b_vec, int b_pp, int b_mp) {
  for (const LayoutVariant& v : kVariants)
    if (v.a_pp == a_pp && v.a_mp == a_mp && v.b_vec == b_vec && v.b_pp == b_pp && v.b_mp == b_mp)
      return &v;
  return nullptr;
}

}  // namespace

bool gemm_layout_supported(int a_pp, int a_mp, int b_vec, int b_pp, int b_mp) {
  return find(a_pp, a_mp, b_vec, b_pp, b_mp) != nullptr;
}

hipError_t launch_gemm_layout(int a_pp, int a_mp, int b_vec, int b_pp, int b_mp, const GemmLaunch& a,
                              hipStream_t s) {
  const LayoutVariant* v = find(a_pp, a_mp, b_vec, b_pp, b_mp);
  if (v == nullptr) return hipErrorInvalidValue;
  return v->launch(a, s);
}

}  // namespace tbl
