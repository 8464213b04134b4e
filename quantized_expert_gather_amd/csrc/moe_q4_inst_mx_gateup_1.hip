// Instantiations of the gate/up kernel over mxfp4 banks, part 1.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU_MX(L_, P_)                                                                    \
  if (lpr == L_ && ppl == P_)                                                                  \
    return full ? (const void*)&k_gateup<L_, P_, true, false, true> : (const void*)&k_gateup<L_, P_, false, false, true>;

const void* gateup_kernel_mx_1(int lpr, int ppl, bool full) {
  MOEQ4_GU_MX(64, 8)
  MOEQ4_GU_MX(32, 1)
  MOEQ4_GU_MX(16, 1)
  MOEQ4_GU_MX(8, 1)
  MOEQ4_GU_MX(4, 1)
  MOEQ4_GU_MX(2, 1)
  return nullptr;
}

}  // namespace moeq4
