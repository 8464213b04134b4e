// Instantiations of the gate/up kernel with matrix-core tiles, part 1.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU_MF(L_, P_)                                                                     \
  if (lpr == L_ && ppl == P_)                                                                  \
    return full ? (const void*)&k_gateup<L_, P_, true, true, kFmtAffine, true>                 \
                : (const void*)&k_gateup<L_, P_, false, true, kFmtAffine, true>;

const void* gateup_kernel_mf_1(int lpr, int ppl, bool full) {
  MOEQ4_GU_MF(64, 6)
  MOEQ4_GU_MF(32, 1)
  MOEQ4_GU_MF(16, 1)
  MOEQ4_GU_MF(8, 1)
  return nullptr;
}

}  // namespace moeq4
