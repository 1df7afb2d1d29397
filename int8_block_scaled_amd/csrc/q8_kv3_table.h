// q8_kv3_table.h -- the 3-bit codec's decision rule as a lookup table.
//
// The code of a binary32 value u is the number of decision thresholds
// t_k <= u, the thresholds being the binary32 midpoints of adjacent levels
// of the 8-level Lloyd-Max quantiser of a unit Gaussian (the format is
// specified in include/q8.h, q8_kv3_encode).  Key the values by their top
// ten bits (sign, exponent, first mantissa bit): each key covers one
// interval of values on which the code rises at most once, so
//
//     code(u) = base[key] + (thr[key] <= u)       (thr NaN: never rises)
//
// for every u that arithmetic can produce (that is, any binary32 value but
// a signalling NaN).  The thresholds +-0.50055, +-1.05 and +-1.748 each fall
// in a key of their own, and t = 0 falls in the key of -0 (code 4 at -0, 3
// just below).  Usable on the host and the device.
#pragma once
#include <stdint.h>

namespace q8 {
namespace kv3 {

constexpr float kLevels[8] = {-2.1520f, -1.3440f, -0.7560f, -0.2451f,
                              0.2451f,  0.7560f,  1.3440f,  2.1520f};

constexpr float threshold(int k) { return (kLevels[k] + kLevels[k + 1]) * 0.5f; }

// the plain rule: number of thresholds t_k <= u (NaN: none)
constexpr int code_count(float u) {
  int c = 0;
  for (int k = 0; k < 7; ++k) c += threshold(k) <= u;
  return c;
}

struct Entry {
  uint32_t base;
  uint32_t thr;   // binary32 bits of the threshold, or a quiet NaN
};

constexpr uint32_t kNaNBits = 0x7fc00000u;

// Entry for key (10 bits).  The key's values form one interval [a, b] (for
// finite keys); the code is constant on it but for at most one threshold
// t with a < t <= b, where it rises by one.
inline __host__ __device__ Entry entry(uint32_t key) {
  const uint32_t sign = key >> 9, lo = key << 22, hi = lo | 0x3fffffu;
  const uint32_t exp_bits = (key >> 1) & 0xffu;
  Entry e{0, kNaNBits};
  if (exp_bits == 0xffu) {                       // inf (and signalling NaNs) or NaN
    e.base = ((key & 1u) == 0 && sign == 0) ? 7u : 0u;
    return e;
  }
  float a, b;                                    // a <= b
  uint32_t ab = sign ? hi : lo, bb = sign ? lo : hi;
  __builtin_memcpy(&a, &ab, 4);
  __builtin_memcpy(&b, &bb, 4);
  e.base = static_cast<uint32_t>(code_count(a));
  for (int k = 0; k < 7; ++k) {
    const float t = threshold(k);
    if (a < t && t <= b) __builtin_memcpy(&e.thr, &t, 4);
  }
  return e;
}

}  // namespace kv3
}  // namespace q8
