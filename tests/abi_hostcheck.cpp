// Host-only driver for the C ABI's argument validation, built by
// tests/test_abi_sanitized.py with g++ and AddressSanitizer +
// UndefinedBehaviorSanitizer together with exact_attention_26_amd/csrc/fa_api.hip
// (compiled as plain C++: its validation makes no HIP call).
//
// The kernel launchers are replaced by stubs that check the problem
// description the entry point built, count the launch and return success, so
// calls that pass validation run the whole host path without a GPU.
//
// Input, one call per line:  <function> <arg> <arg> ...
//   pointers and integers in decimal, floats in C99 hex-float or inf/nan
//   (strtod), NULL as 0. Output, one line per call: "<status> <launches>".
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fa.h"
#include "fa_common.h"

namespace {

int g_launches = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "stub launcher: inconsistent problem description: %s\n", what);
    std::abort();
  }
}

void check_fwd(const fa::FwdParams& p, int rows_per_block) {
  expect(p.q && p.k && p.v && p.o && p.lse, "null tensor");
  expect(p.B > 0 && p.H > 0 && p.N > 0, "empty problem launched");
  expect((int64_t)p.q_blocks * rows_per_block >= p.N, "query blocks do not cover N");
  expect(p.scale > 0.f && std::isfinite(p.scale_log2), "scale");
  expect(p.window >= -1 && p.window <= p.N, "window");
  expect(fa::fwd_grid(p) > 0, "grid");
}

}  // namespace

namespace fa {

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool varlen, hipStream_t) {
  expect(d == 64 || d == 128, "head dim");
  expect(p.key_split == 0 || (!varlen && p.key_split == f32_key_split(d)), "key split");
  const bool small = (int64_t)((p.N + kRowsPerBlockF32 - 1) / kRowsPerBlockF32) * p.H * p.B <
                    kF32SplitBelowBlocks;
  expect(p.key_split == 0 || small, "key split on a large grid");
  expect(p.key_split > 0 || varlen || !small, "small dense fp32 grid without the key split");
  check_fwd(p, p.key_split ? kRowsPerBlockF32Split : kRowsPerBlockF32);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_mfma16(const FwdParams& p, int d, bool, bool, int waves, hipStream_t) {
  expect(d == 64 || d == 128, "head dim");
  expect(p.key_split == 0, "key split outside fp32");
  expect(waves == 4 || waves == 8, "waves");
  check_fwd(p, 32 * waves);
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_kv_outer(const KvOuterParams& p, int d, bool, hipStream_t) {
  expect(d == 64 || d == 128, "head dim");
  expect(p.groups >= 1 && (int64_t)p.groups * p.rows_per_group >= p.N, "query groups");
  expect(p.mstat == p.oacc + (int64_t)p.BH * p.N * d, "m statistics offset");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dropout_add_norm(const NormParams& p, bool, hipStream_t) {
  expect(p.rows > 0 && p.hidden > 0 && p.hidden % 8 == 0, "shape");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams& p, int d, bool, hipStream_t) {
  expect(d == 64 || d == 128, "head dim");
  expect(p.delta != nullptr, "delta");
  expect(p.rows == (int64_t)p.BH * p.N, "rows");
  expect((int64_t)p.kblocks * kBwdKeysPerBlock >= p.N, "key blocks");
  ++g_launches;
  return hipSuccess;
}

hipError_t set_fwd_trace(int, unsigned long long*) { return hipErrorNotSupported; }

}  // namespace fa

namespace {

struct Args {
  std::vector<std::string> v;
  size_t i = 0;
  void* ptr() { return reinterpret_cast<void*>(std::strtoull(v.at(i++).c_str(), nullptr, 10)); }
  long long ll() { return std::strtoll(v.at(i++).c_str(), nullptr, 10); }
  int in() { return (int)ll(); }
  unsigned long long ull() { return std::strtoull(v.at(i++).c_str(), nullptr, 10); }
  float fl() { return (float)std::strtod(v.at(i++).c_str(), nullptr); }
};

int call(const std::string& fn, Args& a) {
  if (fn == "fa_fwd") {
    void *q = a.ptr(), *k = a.ptr(), *v = a.ptr(), *o = a.ptr(), *l = a.ptr();
    int B = a.in(), H = a.in(), N = a.in(), d = a.in();
    float sc = a.fl();
    int dt = a.in();
    void* st = a.ptr();
    return fa_fwd(q, k, v, o, (float*)l, B, H, N, d, sc, dt, st);
  }
  if (fn == "fa_fwd_varlen") {
    void *q = a.ptr(), *k = a.ptr(), *v = a.ptr(), *o = a.ptr(), *l = a.ptr(), *cu = a.ptr();
    int nseq = a.in(), T = a.in(), mx = a.in(), H = a.in(), d = a.in();
    float sc = a.fl();
    int dt = a.in();
    void* st = a.ptr();
    return fa_fwd_varlen(q, k, v, o, (float*)l, (const int32_t*)cu, nseq, T, mx, H, d, sc, dt, st);
  }
  if (fn == "fa_fwd_banded") {
    void *q = a.ptr(), *k = a.ptr(), *v = a.ptr(), *o = a.ptr(), *l = a.ptr();
    int B = a.in(), H = a.in(), N = a.in(), d = a.in(), w = a.in();
    float sc = a.fl();
    int dt = a.in();
    void* st = a.ptr();
    return fa_fwd_banded(q, k, v, o, (float*)l, B, H, N, d, w, sc, dt, st);
  }
  if (fn == "fa_fwd_kv_outer") {
    void *q = a.ptr(), *k = a.ptr(), *v = a.ptr(), *o = a.ptr(), *l = a.ptr(), *acc = a.ptr();
    int B = a.in(), H = a.in(), N = a.in(), d = a.in(), g = a.in();
    float sc = a.fl();
    int dt = a.in();
    void* st = a.ptr();
    return fa_fwd_kv_outer(q, k, v, o, (float*)l, (float*)acc, B, H, N, d, g, sc, dt, st);
  }
  if (fn == "fa_bwd") {
    void* p[10];
    for (auto& x : p) x = a.ptr();
    int B = a.in(), H = a.in(), N = a.in(), d = a.in();
    float sc = a.fl();
    int dt = a.in();
    void* st = a.ptr();
    return fa_bwd(p[0], p[1], p[2], p[3], p[4], (const float*)p[5], p[6], p[7], p[8],
                  (float*)p[9], B, H, N, d, sc, dt, st);
  }
  if (fn == "fa_dropout_add_norm") {
    void* p[13];
    for (auto& x : p) x = a.ptr();
    int rows = a.in(), hidden = a.in();
    float dp = a.fl();
    unsigned long long seed = a.ull(), off = a.ull();
    float eps = a.fl();
    int kind = a.in(), dt = a.in();
    void* st = a.ptr();
    return fa_dropout_add_norm(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9],
                               (float*)p[10], (float*)p[11], (unsigned char*)p[12], rows, hidden,
                               dp, seed, off, eps, kind, dt, st);
  }
  if (fn == "fa_strerror") {
    const char* s = fa_strerror(a.in());
    return (s && std::strlen(s) > 0) ? 0 : -1000;
  }
  if (fn == "fa_version") return fa_version();
  if (fn == "fa_debug_fwd_trace") {
    int wg = a.in();
    void* buf = a.ptr();
    return fa_debug_fwd_trace(wg, (unsigned long long*)buf);
  }
  std::fprintf(stderr, "unknown function %s\n", fn.c_str());
  std::abort();
}

}  // namespace

int main() {
  char line[4096];
  while (std::fgets(line, sizeof line, stdin)) {
    Args a;
    for (char* t = std::strtok(line, " \t\r\n"); t; t = std::strtok(nullptr, " \t\r\n"))
      a.v.emplace_back(t);
    if (a.v.empty()) continue;
    const std::string fn = a.v[0];
    a.i = 1;
    g_launches = 0;
    const int st = call(fn, a);
    std::printf("%d %d\n", st, g_launches);
  }
  return 0;
}
