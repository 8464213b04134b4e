// Kernel pickers of the instantiation units.  Internal header.
#pragma once

namespace moeq4 {

// Host-side handle of the gate/up (down) kernel instantiated for lanes per
// row `lpr`, positions per lane `ppl`, full rows `full`, quad-shared scale
// loads `qs` (and tokens per register pass `nt`); nullptr if not built.
const void* gateup_kernel(int lpr, int ppl, bool full, bool qs);
const void* down_kernel(int lpr, int ppl, bool full, bool qs, int nt);
// the same over mxfp4 banks (E2M1 codes, one E8M0 scale per 32 inputs)
const void* gateup_kernel_mx(int lpr, int ppl, bool full);
const void* down_kernel_mx(int lpr, int ppl, bool full, int nt);

const void* gateup_kernel_0(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_1(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_2(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_3(int lpr, int ppl, bool full, bool qs);
const void* down_kernel_0(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_1(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_2(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_3(int lpr, int ppl, bool full, bool qs, int nt);
const void* gateup_kernel_mx_0(int lpr, int ppl, bool full);
const void* gateup_kernel_mx_1(int lpr, int ppl, bool full);
const void* down_kernel_mx_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_mx_1(int lpr, int ppl, bool full, int nt);

}  // namespace moeq4
