// Host sanitizer driver for the C ABI's host side (argument validation,
// workspace layouts, path selection, status strings), built by
// tests/test_host_sanitizers.py from the library sources compiled for the
// host only, with AddressSanitizer and UndefinedBehaviorSanitizer.  Every call
// below returns from the host-side checks before any HIP runtime call, so no
// GPU is needed; pointers are fake, aligned addresses that are never touched.
// Exit status 0 = clean.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_q4.h"

static int fails = 0;
#define CHECK(c, ...)                        \
  do {                                       \
    if (!(c)) {                              \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");                 \
      ++fails;                               \
    }                                        \
  } while (0)

static void* fake(int i) { return reinterpret_cast<void*>((uintptr_t(1) << 40) + uintptr_t(i) * (uintptr_t(1) << 34)); }
static void* off(void* p, uintptr_t b) { return reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(p) + b); }

struct Call {
  void* p[12];
  int L = 2, k = 2, E = 8, H = 256, I = 128, group = 64, bits = 4, out_dtype = 0;
  void* out = fake(13);
  void* ws = fake(14);
  size_t ws_bytes = size_t(1) << 30;
  unsigned stages = 3;
  Call() {
    for (int i = 0; i < 12; ++i) p[i] = fake(i);
  }
  int run() const {
    return moe_swiglu_q4_forward_stages(p[0], (const int32_t*)p[1], (const float*)p[2], (const uint32_t*)p[3], p[4],
                                        p[5], (const uint32_t*)p[6], p[7], p[8], (const uint32_t*)p[9], p[10], p[11],
                                        L, k, E, H, I, group, bits, out, out_dtype, ws, ws_bytes, stages, nullptr);
  }
  int run_codec(int codec) const {
    return moe_swiglu_codec_forward_stages(codec, p[0], (const int32_t*)p[1], (const float*)p[2],
                                           (const uint32_t*)p[3], p[4], p[5], (const uint32_t*)p[6], p[7], p[8],
                                           (const uint32_t*)p[9], p[10], p[11], L, k, E, H, I, out, out_dtype, ws,
                                           ws_bytes, stages, nullptr);
  }
};

int main() {
  // zero tokens
  {
    Call c;
    c.L = 0;
    CHECK(c.run() == MOE_Q4_OK, "L = 0");
    CHECK(moe_swiglu_q4_workspace_bytes(0, 2, 8, 256, 128) == 0, "ws(L=0)");
    CHECK(moe_swiglu_q4_select_path(0, 2, 8, 256, 128) == MOE_Q4_PATH_NONE, "path(L=0)");
  }
  // invalid shapes and options
  struct { int L, k, E, H, I, g, b, od; unsigned st; size_t wsb; int want; } cases[] = {
      {-1, 2, 8, 256, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_SHAPE},
      {2, 0, 8, 256, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_SHAPE},
      {2, 2, 0, 256, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_SHAPE},
      {2, 9, 8, 256, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_SHAPE},
      {2, 2, 8, 0, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_SHAPE},
      {2, 2, 8, 250, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 96, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 32, 4, 0, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 64, 8, 0, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 64, 4, 5, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 64, 4, 0, 0, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 64, 4, 0, 4, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 20000, 256, 128, 64, 4, 0, 3, 1u << 30, MOE_Q4_ERR_UNSUPPORTED},
      {2, 2, 8, 256, 128, 64, 4, 0, 3, 64, MOE_Q4_ERR_WORKSPACE},
      {600, 8, 64, 1024, 512, 64, 4, 0, 3, 4096, MOE_Q4_ERR_WORKSPACE},  // sorted path, small workspace
  };
  for (const auto& cs : cases) {
    Call c;
    c.L = cs.L; c.k = cs.k; c.E = cs.E; c.H = cs.H; c.I = cs.I; c.group = cs.g; c.bits = cs.b;
    c.out_dtype = cs.od; c.stages = cs.st; c.ws_bytes = cs.wsb;
    const int st = c.run();
    CHECK(st == cs.want, "shape case L=%d k=%d E=%d H=%d I=%d: %d != %d", cs.L, cs.k, cs.E, cs.H, cs.I, st, cs.want);
  }
  // NULL pointers
  for (int i = 0; i < 12; ++i) {
    Call c;
    c.p[i] = nullptr;
    CHECK(c.run() == MOE_Q4_ERR_NULL, "null %d", i);
  }
  {
    Call c;
    c.out = nullptr;
    CHECK(c.run() == MOE_Q4_ERR_NULL, "null out");
    Call d;
    d.ws = nullptr;
    CHECK(d.run() == MOE_Q4_ERR_WORKSPACE, "null workspace");
  }
  // misalignment
  const struct { int i; uintptr_t a; } mis[] = {{0, 8}, {3, 8}, {6, 4}, {9, 2}, {1, 2}, {4, 2}};
  for (const auto& m : mis) {
    Call c;
    c.p[m.i] = off(c.p[m.i], m.a);
    CHECK(c.run() == MOE_Q4_ERR_ALIGN, "align %d", m.i);
  }
  {
    Call c;
    c.ws = off(c.ws, 128);
    CHECK(c.run() == MOE_Q4_ERR_ALIGN, "align ws");
    Call d;
    d.out = off(d.out, 8);
    CHECK(d.run() == MOE_Q4_ERR_ALIGN, "align out");
  }
  // output aliasing an input or the workspace
  {
    Call c;
    c.out = c.p[0];
    CHECK(c.run() == MOE_Q4_ERR_ALIAS, "alias x");
    Call d;
    d.out = off(d.ws, 256);
    CHECK(d.run() == MOE_Q4_ERR_ALIAS, "alias ws");
    Call e;
    e.out = off(e.p[3], 1024);
    CHECK(e.run() == MOE_Q4_ERR_ALIAS, "alias wg");
  }
  // the codec entry point's host checks
  {
    Call c;
    CHECK(c.run_codec(99) == MOE_Q4_ERR_UNSUPPORTED, "unknown codec");
    for (int codec = 1; codec <= 5; ++codec) {
      Call z;
      z.L = 0;
      CHECK(z.run_codec(codec) == MOE_Q4_OK, "codec %d L = 0", codec);
      Call n;
      n.p[3] = nullptr;
      CHECK(n.run_codec(codec) == MOE_Q4_ERR_NULL, "codec %d null wg", codec);
      Call r;
      r.H = 48;
      CHECK(r.run_codec(codec) == MOE_Q4_ERR_UNSUPPORTED, "codec %d H=48", codec);
      Call w;
      w.ws_bytes = 16;
      CHECK(w.run_codec(codec) == MOE_Q4_ERR_WORKSPACE, "codec %d small ws", codec);
      CHECK(moe_swiglu_codec_workspace_bytes(codec, 4, 8, 64, 2048, 512) > 0, "codec %d ws bytes", codec);
      CHECK(moe_swiglu_codec_workspace_bytes(codec, 4, 8, 64, 48, 512) == 0, "codec %d ws bytes of a bad shape", codec);
    }
    // the FP4 / E8M0 codecs ignore the bias slots
    Call b;
    b.p[5] = b.p[8] = b.p[11] = nullptr;
    b.ws = nullptr;
    CHECK(b.run_codec(MOE_Q4_CODEC_MXFP4) == MOE_Q4_ERR_WORKSPACE, "mxfp4 without biases reaches the ws check");
  }
  // path selection and workspace sizes over a sweep of shapes
  const int Ls[] = {1, 2, 3, 8, 31, 32, 33, 128, 512, 2048};
  const int Hs[] = {64, 256, 2048, 4096, 6144, 7168};
  const int Is[] = {64, 128, 512, 2048};
  for (int L : Ls)
    for (int H : Hs)
      for (int I : Is) {
        const int path = moe_swiglu_q4_select_path(L, 8, 256, H, I);
        const size_t n = moe_swiglu_q4_workspace_bytes(L, 8, 256, H, I);
        CHECK(path == MOE_Q4_PATH_UNION || path == MOE_Q4_PATH_SORTED, "path L=%d H=%d I=%d: %d", L, H, I, path);
        CHECK(n > 0 && n % 256 == 0, "ws L=%d H=%d I=%d", L, H, I);
        CHECK(path != MOE_Q4_PATH_UNION || L <= MOE_Q4_UNION_MAX_L, "union past 32 tokens");
      }
  CHECK(moe_swiglu_q4_select_path(64, 8, 16385, 256, 128) == -MOE_Q4_ERR_UNSUPPORTED, "E limit");
  // the allocation-free entry point refuses shapes beyond its scratch on the host
  {
    Call c;
    c.L = 512; c.k = 8; c.E = 16; c.H = 1024; c.I = 256;
    CHECK(moe_swiglu_q4_workspace_bytes(512, 8, 16, 1024, 256) > MOE_Q4_NOALLOC_SCRATCH_BYTES, "scratch case");
    const int st = moe_swiglu_q4_forward_noalloc(c.p[0], (const int32_t*)c.p[1], (const float*)c.p[2],
                                                 (const uint32_t*)c.p[3], c.p[4], c.p[5], (const uint32_t*)c.p[6],
                                                 c.p[7], c.p[8], (const uint32_t*)c.p[9], c.p[10], c.p[11], 512, 8, 16,
                                                 1024, 256, 64, 4, c.out, 0, nullptr);
    CHECK(st == MOE_Q4_ERR_SCRATCH, "noalloc scratch: %d", st);
    CHECK(moe_swiglu_q4_forward_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, nullptr, nullptr, 2, 9, 8, 256, 128, 64, 4, nullptr, 0,
                                        nullptr) == MOE_Q4_ERR_SHAPE, "noalloc shape");
  }
  // route union / sort argument checks
  CHECK(moe_route_union(nullptr, nullptr, 0, 8, 256, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
            MOE_Q4_ERR_SHAPE, "route union L=0");
  CHECK(moe_route_union((const int32_t*)fake(0), (const float*)fake(1), 33, 8, 256, (int32_t*)fake(2),
                        (int32_t*)fake(3), (uint32_t*)fake(4), (float*)fake(5), (int32_t*)fake(6), nullptr) ==
            MOE_Q4_ERR_UNSUPPORTED, "route union L=33");
  CHECK(moe_sort_pairs_tiles_max(100, 8, 256, 32) == 100 * 8 / 32 + 256 + 1, "tiles max");
  CHECK(moe_sort_pairs(nullptr, 10, 2, 8, 32, nullptr, nullptr, nullptr, nullptr, 1000, nullptr, nullptr,
                       nullptr) == MOE_Q4_ERR_NULL, "sort null");
  // status strings
  for (int s = -2; s <= 12; ++s) {
    const char* str = moe_q4_status_string(s);
    CHECK(str && strlen(str) > 0, "status string %d", s);
  }
  if (fails) {
    fprintf(stderr, "%d check(s) failed\n", fails);
    return 1;
  }
  printf("ABI host sanitizer driver: all checks passed\n");
  return 0;
}
