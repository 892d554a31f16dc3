// Replays recorded C-ABI calls against a host-only build of fa_api.hip (the
// kernel launchers replaced by stand-ins) and checks that each call returns
// the recorded result.  Built with AddressSanitizer and UndefinedBehavior-
// Sanitizer, so any out-of-bounds access or undefined arithmetic on the way
// (for instance a signed overflow in a size product) aborts the run.
//
// Input: one call per line, "<function> <arg> ... => <result>".  Integers are
// decimal (pointers as addresses, 0 for NULL), floats carry a trailing 'f'
// ("0.125f", "nanf", "inff").
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>
#include <vector>

#include "fa.h"

namespace {

struct Args {
  std::vector<std::string> v;
  size_t i = 0;
  const std::string& next() {
    if (i >= v.size()) {
      std::fprintf(stderr, "too few arguments\n");
      std::exit(2);
    }
    return v[i++];
  }
  long long I() { return std::stoll(next()); }
  void* P() { return reinterpret_cast<void*>(static_cast<uintptr_t>(std::stoull(next()))); }
  float F() {
    std::string s = next();
    if (!s.empty() && s.back() == 'f') s.pop_back();
    return std::strtof(s.c_str(), nullptr);
  }
  fa_dtype D() { return static_cast<fa_dtype>(I()); }
  hipStream_t S() { return static_cast<hipStream_t>(P()); }
};

long long call(const std::string& fn, Args& a) {
  if (fn == "fa_fwd") {
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P();
    float sc = a.F();
    int ca = (int)a.I();
    void* O = a.P();
    float* L = (float*)a.P();
    return fa_fwd(it, ot, B, H, Lq, Lk, d, Q, K, V, sc, ca, O, L, a.S());
  }
  if (fn == "fa_fwd_blocksparse") {
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P();
    float sc = a.F();
    int ca = (int)a.I();
    const uint8_t* m = (const uint8_t*)a.P();
    long long ns = a.I();
    void* O = a.P();
    float* L = (float*)a.P();
    return fa_fwd_blocksparse(it, ot, B, H, Lq, Lk, d, Q, K, V, sc, ca, m, ns, O, L, a.S());
  }
  if (fn == "fa_bwd" || fn == "fa_bwd_blocksparse") {
    const bool bs = fn == "fa_bwd_blocksparse";
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P(), *O = a.P(), *G = a.P();
    const float* L = (const float*)a.P();
    float sc = a.F();
    int ca = (int)a.I();
    const uint8_t* m = nullptr;
    long long ns = 0;
    if (bs) {
      m = (const uint8_t*)a.P();
      ns = a.I();
    }
    void *dQ = a.P(), *dK = a.P(), *dV = a.P(), *ws = a.P();
    size_t wb = (size_t)a.I();
    hipStream_t s = a.S();
    if (bs) return fa_bwd_blocksparse(it, ot, B, H, Lq, Lk, d, Q, K, V, O, G, L, sc, ca, m, ns, dQ, dK, dV, ws, wb, s);
    return fa_bwd(it, ot, B, H, Lq, Lk, d, Q, K, V, O, G, L, sc, ca, dQ, dK, dV, ws, wb, s);
  }
  if (fn == "fa_bwd_noalloc") {
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P(), *O = a.P(), *G = a.P();
    const float* L = (const float*)a.P();
    float sc = a.F();
    int ca = (int)a.I();
    void *dQ = a.P(), *dK = a.P(), *dV = a.P();
    return fa_bwd_noalloc(it, ot, B, H, Lq, Lk, d, Q, K, V, O, G, L, sc, ca, dQ, dK, dV, a.S());
  }
  if (fn == "fa_bwd_prepare_dq") {
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P(), *O = a.P(), *G = a.P();
    const float* L = (const float*)a.P();
    float sc = a.F();
    int ca = (int)a.I();
    void* dQ = a.P();
    void* ws = a.P();
    size_t wb = (size_t)a.I();
    return fa_bwd_prepare_dq(it, ot, B, H, Lq, Lk, d, Q, K, V, O, G, L, sc, ca, dQ, ws, wb, a.S());
  }
  if (fn == "fa_bwd_prepare") {
    fa_dtype it = a.D(), ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *O = a.P(), *G = a.P();
    const float* L = (const float*)a.P();
    void* ws = a.P();
    size_t wb = (size_t)a.I();
    return fa_bwd_prepare(it, ot, B, H, Lq, Lk, d, O, G, L, ws, wb, a.S());
  }
  if (fn == "fa_bwd_dkdv" || fn == "fa_bwd_dq") {
    fa_dtype it = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P(), *G = a.P();
    float sc = a.F();
    int ca = (int)a.I();
    if (fn == "fa_bwd_dkdv") {
      void *dK = a.P(), *dV = a.P(), *ws = a.P();
      size_t wb = (size_t)a.I();
      return fa_bwd_dkdv(it, B, H, Lq, Lk, d, Q, K, V, G, sc, ca, dK, dV, ws, wb, a.S());
    }
    void *dQ = a.P(), *ws = a.P();
    size_t wb = (size_t)a.I();
    return fa_bwd_dq(it, B, H, Lq, Lk, d, Q, K, V, G, sc, ca, dQ, ws, wb, a.S());
  }
  if (fn == "fa_bwd_workspace_bytes") {
    fa_dtype it = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    return (long long)fa_bwd_workspace_bytes(it, B, H, Lq, Lk, d);
  }
  if (fn == "fa_fwd_splitkv" || fn == "fa_fwd_splitkv_partial") {
    const bool full = fn == "fa_fwd_splitkv";
    fa_dtype it = a.D(), ot = full ? a.D() : FA_BF16;
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    void *Q = a.P(), *K = a.P(), *V = a.P();
    float sc = a.F();
    int ca = (int)a.I();
    long long ns = a.I();
    void *O = nullptr, *L = nullptr;
    if (full) {
      O = a.P();
      L = a.P();
    }
    void* ws = a.P();
    size_t wb = (size_t)a.I();
    hipStream_t s = a.S();
    if (full) return fa_fwd_splitkv(it, ot, B, H, Lq, Lk, d, Q, K, V, sc, ca, ns, O, (float*)L, ws, wb, s);
    return fa_fwd_splitkv_partial(it, B, H, Lq, Lk, d, Q, K, V, sc, ca, ns, ws, wb, s);
  }
  if (fn == "fa_fwd_splitkv_merge") {
    fa_dtype ot = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), d = a.I(), ns = a.I();
    void* ws = a.P();
    size_t wb = (size_t)a.I();
    void* O = a.P();
    float* L = (float*)a.P();
    return fa_fwd_splitkv_merge(ot, B, H, Lq, d, ns, ws, wb, O, L, a.S());
  }
  if (fn == "fa_fwd_splitkv_workspace_bytes") {
    fa_dtype it = a.D();
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I(), ns = a.I();
    return (long long)fa_fwd_splitkv_workspace_bytes(it, B, H, Lq, Lk, d, ns);
  }
  if (fn == "fa_fwd_splitkv_default_splits") {
    long long B = a.I(), H = a.I(), Lq = a.I(), Lk = a.I(), d = a.I();
    return fa_fwd_splitkv_default_splits(B, H, Lq, Lk, d);
  }
  if (fn == "fa_bwd_noalloc_max_scratch_bytes") return (long long)fa_bwd_noalloc_max_scratch_bytes();
  if (fn == "fa_status_str") return (long long)std::strlen(fa_status_str((fa_status)a.I()));
  if (fn == "fa_version") return (long long)std::strlen(fa_version());
  std::fprintf(stderr, "unknown function %s\n", fn.c_str());
  std::exit(2);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: replay CALLS\n");
    return 2;
  }
  std::ifstream in(argv[1]);
  std::string line;
  int n = 0, bad = 0;
  while (std::getline(in, line)) {
    if (line.empty()) continue;
    std::istringstream ss(line);
    std::string fn, tok;
    ss >> fn;
    Args a;
    long long want = 0;
    while (ss >> tok) {
      if (tok == "=>") {
        ss >> want;
        break;
      }
      a.v.push_back(tok);
    }
    const long long got = call(fn, a);
    ++n;
    if (got != want) {
      ++bad;
      std::fprintf(stderr, "mismatch: %s -> %lld, recorded %lld\n", line.c_str(), got, want);
    }
  }
  std::printf("%d calls replayed, %d mismatches\n", n, bad);
  return bad == 0 && n > 0 ? 0 : 1;
}
