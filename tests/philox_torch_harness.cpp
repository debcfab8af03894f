// Test harness: prints Philox4x32-10 words from PyTorch's header-only engine so the
// oracle's generator can be checked against an independent implementation.
// Usage: harness <seed> <subsequence> <offset>  -> four hex words (one 128-bit block)
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  uint64_t seed = std::strtoull(argv[1], nullptr, 0);
  uint64_t sub = std::strtoull(argv[2], nullptr, 0);
  uint64_t off = std::strtoull(argv[3], nullptr, 0);
  at::Philox4_32 eng(seed, sub, off);
  for (int i = 0; i < 4; ++i) std::printf("%08x\n", static_cast<unsigned>(eng()));
  return 0;
}
