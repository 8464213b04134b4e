// Instantiations of the gate/up kernel, part 0.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_GU(L_, P_)                                                                              \
  if (lpr == L_ && ppl == P_) {                                                                       \
    if (full) return qs ? (const void*)&k_gateup<L_, P_, true, (L_ >= 4)> : (const void*)&k_gateup<L_, P_, true, false>; \
    return qs ? (const void*)&k_gateup<L_, P_, false, (L_ >= 4)> : (const void*)&k_gateup<L_, P_, false, false>;       \
  }

const void* gateup_kernel_0(int lpr, int ppl, bool full, bool qs) {
  MOEQ4_GU(64, 1)
  MOEQ4_GU(64, 2)
  return nullptr;
}

}  // namespace moeq4
