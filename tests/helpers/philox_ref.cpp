// Test helper: prints rocRAND's Philox4x32-10 output blocks (host-side inline
// functions of the installed rocRAND headers; no GPU is touched).  Used only to
// pin the CPU oracle's own Philox implementation to an independent library.
// stdin: lines "seed subsequence offset"; stdout: four hex words per line.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    const uint4 v = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
