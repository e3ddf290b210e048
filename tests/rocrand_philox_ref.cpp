// Reference Philox4x32-10 words from ROCm's rocRAND device library, run on the
// host.  Test infrastructure: pins the oracle's Philox against an independent
// library implementation of the same published generator (Salmon et al., SC'11).
//
// stdin : lines "seed_hex c0 c1 c2 c3" (counter words, hex)
// stdout: the four 32-bit output words of that counter under key = seed, hex.
//
// rocRAND keys the generator with (seed low, seed high); `subsequence` fills
// counter words 2..3, and skipping ahead by 4 n outputs adds n to counter
// words 0..1 (done in steps so that 4 n never overflows 64 bits).
#include <cstdio>
#include <cstdint>
#include <rocrand/rocrand_kernel.h>

int main() {
  unsigned long long seed;
  unsigned c0, c1, c2, c3;
  while (std::scanf("%llx %x %x %x %x", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    const unsigned long long subsequence =
        (static_cast<unsigned long long>(c3) << 32) | c2;
    unsigned long long n = (static_cast<unsigned long long>(c1) << 32) | c0;
    rocrand_init(seed, subsequence, 0ull, &st);
    while (n > 0) {
      const unsigned long long m = n < (1ull << 61) ? n : (1ull << 61);
      skipahead(4ull * m, &st);
      n -= m;
    }
    const uint4 v = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
