// Exhaustive host check of the 3-bit codec's decision table
// (int8_block_scaled_amd/csrc/q8_kv3_table.h) against the plain rule, the
// number of thresholds t_k <= u, with the seven thresholds given on the
// command line as binary32 bit patterns (taken from the oracle's codebook by
// the calling test).  Every binary32 u except the signalling NaNs, which no
// arithmetic produces.  Exits non-zero and prints the first mismatches.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#define __host__
#define __device__
#include "q8_kv3_table.h"

int main(int argc, char** argv) {
  if (argc != 8) return 2;
  float t[7];
  for (int k = 0; k < 7; ++k) {
    const unsigned long b = std::strtoul(argv[k + 1], nullptr, 16);
    const unsigned int bits = static_cast<unsigned int>(b);
    std::memcpy(&t[k], &bits, 4);
  }
  q8::kv3::Entry table[1024];
  for (unsigned key = 0; key < 1024; ++key) table[key] = q8::kv3::entry(key);
  long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long long i = 0; i < (1LL << 32); ++i) {
    const unsigned int bits = static_cast<unsigned int>(i);
    const bool nan = (bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0;
    if (nan && (bits & 0x00400000u) == 0) continue;            // signalling NaN
    float u;
    std::memcpy(&u, &bits, 4);
    int want = 0;
    for (int k = 0; k < 7; ++k) want += t[k] <= u;
    const q8::kv3::Entry e = table[bits >> 22];
    float thr;
    std::memcpy(&thr, &e.thr, 4);
    const int got = static_cast<int>(e.base) + (thr <= u ? 1 : 0);
    if (got != want) {
      if (bad < 5) std::printf("mismatch u bits %08x: table %d, rule %d\n", bits, got, want);
      ++bad;
    }
  }
  std::printf("checked 2^32 binary32 values (signalling NaNs excepted): %lld mismatches\n", bad);
  return bad ? 1 : 0;
}
