// Instantiations of the down kernel over mxfp4 banks, part 1.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_DN_MX_NT(L_, P_, F_) \
  (nt == 1 ? (const void*)&k_down<L_, P_, F_, false, 1, true> : (const void*)&k_down<L_, P_, F_, false, 2, true>)
#define MOEQ4_DN_MX(L_, P_) \
  if (lpr == L_ && ppl == P_) return full ? MOEQ4_DN_MX_NT(L_, P_, true) : MOEQ4_DN_MX_NT(L_, P_, false);

const void* down_kernel_mx_1(int lpr, int ppl, bool full, int nt) {
  MOEQ4_DN_MX(32, 1)
  MOEQ4_DN_MX(16, 1)
  MOEQ4_DN_MX(8, 1)
  MOEQ4_DN_MX(4, 1)
  MOEQ4_DN_MX(2, 1)
  return nullptr;
}

}  // namespace moeq4
