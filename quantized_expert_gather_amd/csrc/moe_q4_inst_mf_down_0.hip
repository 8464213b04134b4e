// Instantiations of the down kernel with matrix-core tiles (512-thread
// blocks: two tokens per register pass at one position per lane, one token
// at two).
#include "moe_q4_inst.h"
#include "moe_q4_union_kernels.h"

namespace moeq4 {

#define MOEQ4_DN_MF(L_, P_, N_)                                                                 \
  if (lpr == L_ && ppl == P_ && nt == N_)                                                      \
    return full ? (const void*)&k_down<L_, P_, true, true, N_, kFmtAffine, true>               \
                : (const void*)&k_down<L_, P_, false, true, N_, kFmtAffine, true>;

const void* down_kernel_mf_0(int lpr, int ppl, bool full, int nt) {
  MOEQ4_DN_MF(64, 1, 2)
  MOEQ4_DN_MF(64, 2, 1)
  MOEQ4_DN_MF(32, 1, 2)
  MOEQ4_DN_MF(16, 1, 2)
  MOEQ4_DN_MF(8, 1, 2)
  return nullptr;
}

}  // namespace moeq4
