// LDS-layout variants of the 256 x 256 fp16 -> fp16 GEMM (kernel in gemm_pp_kernel.hpp), in its
// 32 x 32 x 16 form and in the default kernel's 16 x 16 x 32 form.
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

// The 16 x 16 x 32 form (the default kernel's MFMA shape and read patterns): b_vec = 0 is its
// default B layout, chunk XOR 4 (k mod 4) + 2 ((k / 8) mod 2); the first entry is the default kernel.
template <int kAPP, int kAMP, int kBV, int kBPP, int kBMP>
hipError_t launch16(const GemmLaunch& a, hipStream_t s) {
  return launch_pp_typed<false, false, kAPP, kAMP, kBV, kBPP, kBMP, false, true>(a, s);
}

constexpr LayoutVariant kVariants16[] = {
    {2, 4, 0, 0, 0, &launch16<2, 4, 0, 0, 0>},   // the default layouts
    {4, 4, 0, 0, 0, &launch16<4, 4, 0, 0, 0>},
    {1, 1, 0, 0, 0, &launch16<1, 1, 0, 0, 0>},   // A unswizzled
    {4, 2, 0, 0, 0, &launch16<4, 2, 0, 0, 0>},
    {2, 4, 4, 1, 4, &launch16<2, 4, 4, 1, 4>},   // B: the 32 x 32 x 16 form's layout
    {2, 4, 1, 1, 1, &launch16<2, 4, 1, 1, 1>},   // B unswizzled
};

template <size_t N>
const LayoutVariant* find_in(const LayoutVariant (&table)[N], int a_pp, int a_mp, int b_vec, int b_pp,
                             int b_mp) {
  for (const LayoutVariant& v : table)
    if (v.a_pp == a_pp && v.a_mp == a_mp && v.b_vec == b_vec && v.b_pp == b_pp && v.b_mp == b_mp)
      return &v;
  return nullptr;
}

const LayoutVariant* find(bool m16, int a_pp, int a_mp, int b_vec, int b_pp, int b_mp) {
  return m16 ? find_in(kVariants16, a_pp, a_mp, b_vec, b_pp, b_mp)
             : find_in(kVariants, a_pp, a_mp, b_vec, b_pp, b_mp);
}

}  // namespace

bool gemm_layout_supported(bool m16, int a_pp, int a_mp, int b_vec, int b_pp, int b_mp) {
  return find(m16, a_pp, a_mp, b_vec, b_pp, b_mp) != nullptr;
}

hipError_t launch_gemm_layout(bool m16, int a_pp, int a_mp, int b_vec, int b_pp, int b_mp,
                              const GemmLaunch& a, hipStream_t s) {
  const LayoutVariant* v = find(m16, a_pp, a_mp, b_vec, b_pp, b_mp);
  if (v == nullptr) return hipErrorInvalidValue;
  return v->launch(a, s);
}

}  // namespace tbl
