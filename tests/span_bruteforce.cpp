// Brute-force check of rmsn_host::overlap (the aliasing test of the C ABI):
// random row-strided spans inside a small address window, each span's bytes
// marked in a bitmap, the exact answer compared with overlap().  overlap()
// must never miss a shared byte, and must be exact when both spans have
// several rows of one pitch no shorter than either row (rows interleave).
// Prints "ok <cases> <exact cases>" or the first failing case; exit status 1
// on failure.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmsnorm_span.hpp"

using rmsn_host::overlap;
using rmsn_host::Span;

static unsigned long long state = 0x9e3779b97f4a7c15ull;
static unsigned rnd(unsigned n) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (unsigned)((state >> 33) % n);
}

int main(int argc, char** argv) {
  const long cases = argc > 1 ? atol(argv[1]) : 200000;
  static unsigned char mark[1 << 14];
  char* const base = (char*)0x100000;  // never dereferenced
  long exact = 0;
  for (long c = 0; c < cases; ++c) {
    Span s[2];
    const int64_t pitch = 1 + rnd(64);
    for (int q = 0; q < 2; ++q) {
      s[q].rows = 1 + rnd(12);
      s[q].pitch = rnd(4) ? pitch : 1 + rnd(64);  // mostly one shared pitch
      s[q].len = 1 + rnd(rnd(2) ? (unsigned)s[q].pitch : 80u);
      s[q].base = base + rnd(2048);
    }
    memset(mark, 0, sizeof mark);
    bool shared = false;
    for (int q = 0; q < 2; ++q)
      for (int64_t r = 0; r < s[q].rows; ++r)
        for (int64_t b = 0; b < s[q].len; ++b) {
          const int64_t at = ((const char*)s[q].base - base) + r * s[q].pitch + b;
          if (q == 0) mark[at] = 1;
          else if (mark[at]) shared = true;
        }
    const bool got = overlap(s[0], s[1]);
    const bool is_exact = s[0].pitch == s[1].pitch && s[0].rows > 1 && s[1].rows > 1 &&
                          s[0].pitch >= s[0].len && s[0].pitch >= s[1].len;
    exact += is_exact;
    if ((shared && !got) || (is_exact && got != shared)) {
      printf("FAIL case %ld: a{base+%ld pitch %ld len %ld rows %ld} b{base+%ld pitch %ld len %ld "
             "rows %ld}: shared %d overlap() %d\n",
             c, (long)((const char*)s[0].base - base), (long)s[0].pitch, (long)s[0].len,
             (long)s[0].rows, (long)((const char*)s[1].base - base), (long)s[1].pitch,
             (long)s[1].len, (long)s[1].rows, shared, got);
      return 1;
    }
  }
  printf("ok %ld %ld\n", cases, exact);
  return 0;
}
