// Prints the 32-bit words of rocRAND's Philox4x32-10 engine, host side.
// Test helper: an implementation of Philox independent of the oracle, used to
// pin the oracle's stochastic-rounding stream.
// usage: rocrand_philox_words SEED SUBSEQUENCE OFFSET COUNT
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  unsigned long long sub = std::strtoull(argv[2], nullptr, 0);
  unsigned long long off = std::strtoull(argv[3], nullptr, 0);
  long n = std::strtol(argv[4], nullptr, 0);
  rocrand_device::philox4x32_10_engine eng(seed, sub, off);
  for (long i = 0; i < n; ++i) std::printf("%u\n", eng());
  return 0;
}
