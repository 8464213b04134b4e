// Instantiations of the gate/up kernel over mxfp8 banks, part 1.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU_F(L_, P_)                                                                           \
  if (lpr == L_ && ppl == P_)                                                                        \
    return full ? (const void*)&k_gateup<L_, P_, true, false, kFmtMxfp8> : (const void*)&k_gateup<L_, P_, false, false, kFmtMxfp8>;

const void* gateup_kernel_mxfp8_1(int lpr, int ppl, bool full) {
  MOEQ4_GU_F(64, 8)
  MOEQ4_GU_F(32, 1)
  MOEQ4_GU_F(16, 1)
  MOEQ4_GU_F(8, 1)
  MOEQ4_GU_F(4, 1)
  MOEQ4_GU_F(2, 1)
  return nullptr;
}

}  // namespace moeq4
