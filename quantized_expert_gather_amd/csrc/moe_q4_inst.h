// Kernel pickers of the instantiation units.  Internal header.
#pragma once

namespace moeq4 {

// Host-side handle of the gate/up (down) kernel instantiated for lanes per
// row `lpr`, positions per lane `ppl`, full rows `full`, quad-shared scale
// loads `qs` (and tokens per register pass `nt`); nullptr if not built.
const void* gateup_kernel(int lpr, int ppl, bool full, bool qs);
const void* down_kernel(int lpr, int ppl, bool full, bool qs, int nt);

const void* gateup_kernel_0(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_1(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_2(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_3(int lpr, int ppl, bool full, bool qs);
const void* down_kernel_0(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_1(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_2(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_3(int lpr, int ppl, bool full, bool qs, int nt);

}  // namespace moeq4
