// Instantiations of the gate/up kernel over 8-bit affine banks (group 64), part 0.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU_F(L_, P_)                                                                           \
  if (lpr == L_ && ppl == P_)                                                                        \
    return full ? (const void*)&k_gateup<L_, P_, true, false, kFmtAffine8> : (const void*)&k_gateup<L_, P_, false, false, kFmtAffine8>;

const void* gateup_kernel_affine8_0(int lpr, int ppl, bool full) {
  MOEQ4_GU_F(64, 1)
  MOEQ4_GU_F(64, 2)
  MOEQ4_GU_F(64, 3)
  MOEQ4_GU_F(64, 4)
  MOEQ4_GU_F(64, 6)
  return nullptr;
}

}  // namespace moeq4
