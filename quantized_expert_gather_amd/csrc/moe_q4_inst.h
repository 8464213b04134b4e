// Kernel pickers of the instantiation units.  Internal header.
#pragma once

namespace moeq4 {

// Host-side handle of the gate/up (down) kernel instantiated for lanes per
// row `lpr`, positions per lane `ppl`, full rows `full`, quad-shared scale
// loads `qs` (and tokens per register pass `nt`); nullptr if not built.
const void* gateup_kernel(int lpr, int ppl, bool full, bool qs);
const void* down_kernel(int lpr, int ppl, bool full, bool qs, int nt);
// matrix-core instances (4-bit affine group 64, quad-shared scale loads;
// at most 6 positions per lane for gate/up, 2 for down; nullptr past what is
// built, and the launch takes the plain instance)
const void* gateup_kernel_mf(int lpr, int ppl, bool full);
const void* down_kernel_mf(int lpr, int ppl, bool full, int nt);
const void* gateup_kernel_mf_0(int lpr, int ppl, bool full);
const void* gateup_kernel_mf_1(int lpr, int ppl, bool full);
const void* down_kernel_mf_0(int lpr, int ppl, bool full, int nt);
// the same for the other weight formats (kFmt*; no quad-shared scale loads)
const void* gateup_kernel_fmt(int fmt, int lpr, int ppl, bool full);
const void* down_kernel_fmt(int fmt, int lpr, int ppl, bool full, int nt);

const void* gateup_kernel_0(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_1(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_2(int lpr, int ppl, bool full, bool qs);
const void* gateup_kernel_3(int lpr, int ppl, bool full, bool qs);
const void* down_kernel_0(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_1(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_2(int lpr, int ppl, bool full, bool qs, int nt);
const void* down_kernel_3(int lpr, int ppl, bool full, bool qs, int nt);
const void* gateup_kernel_mxfp4_0(int lpr, int ppl, bool full);
const void* gateup_kernel_mxfp4_1(int lpr, int ppl, bool full);
const void* down_kernel_mxfp4_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_mxfp4_1(int lpr, int ppl, bool full, int nt);
const void* gateup_kernel_nvfp4_0(int lpr, int ppl, bool full);
const void* gateup_kernel_nvfp4_1(int lpr, int ppl, bool full);
const void* down_kernel_nvfp4_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_nvfp4_1(int lpr, int ppl, bool full, int nt);
const void* gateup_kernel_affine32_0(int lpr, int ppl, bool full);
const void* gateup_kernel_affine32_1(int lpr, int ppl, bool full);
const void* down_kernel_affine32_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_affine32_1(int lpr, int ppl, bool full, int nt);
const void* gateup_kernel_affine8_0(int lpr, int ppl, bool full);
const void* gateup_kernel_affine8_1(int lpr, int ppl, bool full);
const void* down_kernel_affine8_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_affine8_1(int lpr, int ppl, bool full, int nt);
const void* gateup_kernel_mxfp8_0(int lpr, int ppl, bool full);
const void* gateup_kernel_mxfp8_1(int lpr, int ppl, bool full);
const void* down_kernel_mxfp8_0(int lpr, int ppl, bool full, int nt);
const void* down_kernel_mxfp8_1(int lpr, int ppl, bool full, int nt);

}  // namespace moeq4
