// Instantiations of the down kernel, part 2.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_DN_NT(L_, P_, F_, N_)                                                   \
  (qs ? (const void*)&k_down<L_, P_, F_, (L_ >= 4), N_> : (const void*)&k_down<L_, P_, F_, false, N_>)
#define MOEQ4_DN(L_, P_)                                                              \
  if (lpr == L_ && ppl == P_) {                                                       \
    if (full) return nt == 1 ? MOEQ4_DN_NT(L_, P_, true, 1) : MOEQ4_DN_NT(L_, P_, true, 2);   \
    return nt == 1 ? MOEQ4_DN_NT(L_, P_, false, 1) : MOEQ4_DN_NT(L_, P_, false, 2);           \
  }

const void* down_kernel_2(int lpr, int ppl, bool full, bool qs, int nt) {
  MOEQ4_DN(32, 1)
  MOEQ4_DN(16, 1)
  return nullptr;
}

}  // namespace moeq4
