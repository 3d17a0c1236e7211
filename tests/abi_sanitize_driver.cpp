// Driver for the sanitizer run of the library's host code (tests/test_sanitizers.py builds
// nonuniform_fft_amd/csrc/plan.cpp with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host side only and links it with the library's other objects).  It calls every C ABI entry
// point on the argument-checking paths that return before any device call: null handles and
// pointers, invalid types, dimensions, mode counts, tolerances, precisions and upsampling
// factors, and every status string.  Exit status 0 = all checks passed.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include "nufft_amd.h"
int main() {
  int fails = 0;
  auto chk = [&](bool c, const char* w) { if (!c) { std::fprintf(stderr, "FAIL %s\n", w); ++fails; } };
  chk(nufft_default_opts(nullptr) == NUFFT_ERR_BAD_ARG, "opts null");
  nufft_opts o; chk(nufft_default_opts(&o) == 0 && o.method == 0, "opts");
  chk(nufft_destroy(nullptr) == 0, "destroy null");
  int64_t N[3] = {16, 16, 16}, Nbad[3] = {16, 0, 16};
  nufft_plan h = nullptr;
  struct { int t, d; const int64_t* n; double e; int p; } bad[] = {
    {4,2,N,1e-5,0},{0,2,N,1e-5,0},{1,4,N,1e-5,0},{1,0,N,1e-5,0},{1,2,N,0.0,0},{1,2,N,-1.0,0},
    {1,2,N,NAN,0},{1,2,N,1e-5,2},{1,2,nullptr,1e-5,0},{2,3,Nbad,1e-5,1},{1,2,N,INFINITY,0}};
  for (auto& b : bad) { chk(nufft_plan_create(b.t, b.d, b.n, b.e, b.p, nullptr, nullptr, &h) == NUFFT_ERR_BAD_ARG && !h, "bad plan"); }
  chk(nufft_plan_create(1, 2, N, 1e-5, 0, nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "null out");
  for (double s : {1.1, 2.5, -1.0, (double)NAN}) { nufft_default_opts(&o); o.upsampfac = s;
    chk(nufft_plan_create(1, 2, N, 1e-5, 0, nullptr, &o, &h) == NUFFT_ERR_BAD_ARG && !h, "sigma"); }
  for (int c : {0, 1, -1, -2, -3, -4, -5, -6, -7, 12345}) chk(nufft_strerror(c) && std::strlen(nufft_strerror(c)) > 0, "strerror");
  chk(std::strcmp(nufft_last_error(nullptr), "") == 0, "last_error null");
  chk(nufft_setpts(nullptr, 0, nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "setpts null");
  chk(nufft_execute(nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "execute null");
  chk(nufft_spread(nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "spread null");
  chk(nufft_interp(nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "interp null");
  chk(nufft_get_info(nullptr, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "info null");
  double ms[8]; chk(nufft_get_stage_times(nullptr, ms) == NUFFT_ERR_BAD_ARG, "times null");
  chk(nufft_execute_many(nullptr, 1, nullptr, nullptr) == NUFFT_ERR_BAD_ARG, "many null");
  std::printf(fails ? "failures\n" : "host ABI sanitizer run: all checks passed\n");
  return fails ? 1 : 0;
}
