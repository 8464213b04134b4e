// Instantiations of the down kernel over mxfp8 banks, part 0.
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_DN_F_NT(L_, P_, F_) \
  (nt == 1 ? (const void*)&k_down<L_, P_, F_, false, 1, kFmtMxfp8> : (const void*)&k_down<L_, P_, F_, false, 2, kFmtMxfp8>)
#define MOEQ4_DN_F(L_, P_) \
  if (lpr == L_ && ppl == P_) return full ? MOEQ4_DN_F_NT(L_, P_, true) : MOEQ4_DN_F_NT(L_, P_, false);

const void* down_kernel_mxfp8_0(int lpr, int ppl, bool full, int nt) {
  MOEQ4_DN_F(64, 1)
  MOEQ4_DN_F(64, 2)
  MOEQ4_DN_F(64, 4)
  return nullptr;
}

}  // namespace moeq4
