// Instantiations of the gate/up kernel with matrix-core tiles, part 0.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU_MF(L_, P_)                                                                     \
  if (lpr == L_ && ppl == P_)                                                                  \
    return full ? (const void*)&k_gateup<L_, P_, true, true, kFmtAffine, true>                 \
                : (const void*)&k_gateup<L_, P_, false, true, kFmtAffine, true>;

const void* gateup_kernel_mf_0(int lpr, int ppl, bool full) {
  MOEQ4_GU_MF(64, 1)
  MOEQ4_GU_MF(64, 2)
  MOEQ4_GU_MF(64, 3)
  MOEQ4_GU_MF(64, 4)
  return nullptr;
}

}  // namespace moeq4
