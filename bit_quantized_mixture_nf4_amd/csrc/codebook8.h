// codebook8.h -- the 128 ascending magnitudes of the two 8-bit storage lanes,
// computed at compile time (host and device code).
//
// The 0.4.0 README's storage-modes support matrix names the lanes: int8, a
// "blockwise dynamic map", and fp8, an "e4m3 codebook"; it prints neither
// table. A code is sign bit 7 | index bits 6..0 into the magnitudes below,
// scaled by the block absmax like the 4-bit codebooks.
//  * fp8: the E4M3 bit patterns 0..127 read with exponent bias 7, subnormals
//    at exponent 0 and no reserved NaN pattern (a codebook, so the top
//    pattern is 1.875 * 2^8 = 480), divided by 480.
//  * int8: the dynamic tree map of block-wise 8-bit quantization (Dettmers et
//    al., "8-bit Optimizers via Block-wise Quantization", arXiv:2110.02861,
//    section "Dynamic Tree Quantization"): after the sign, z leading zeros set
//    the decimal exponent 10^-z, the first one bit is the indicator, and the
//    remaining n = 6 - z bits f choose the linear fraction
//    0.1 + 0.9 (f + 1) / 2^n of [0.1, 1]; with the all-zero pattern as 0, 128
//    magnitudes from 10^-6 to 1, stored by ascending rank.
// Every magnitude is an exact rational rounded once to fp32 (nearest even),
// by integer arithmetic, so the tables are exactly the same on every
// compiler and both sides of the build.
#pragma once

#include <stdint.h>

namespace e4b {

// fp32 nearest (ties to even) to num * 2^sh / den, for a value in the normal
// range; integer arithmetic only.
constexpr float f32_of_ratio(uint64_t num, int sh, uint64_t den) {
  // q = floor(num * 2^k / den) in [2^23, 2^24), value = q * 2^(sh - k)
  unsigned __int128 n = num, d = den;
  int k = 0;
  while ((n << k) < (d << 23)) ++k;
  while ((n << k) >= (d << 24)) --k;  // k may go negative only for values >= 2^24
  unsigned __int128 nk = k >= 0 ? (n << k) : n;
  unsigned __int128 dk = k >= 0 ? d : (d << -k);
  uint64_t q = uint64_t(nk / dk);
  const unsigned __int128 r = nk - dk * q;
  if (2 * r > dk || (2 * r == dk && (q & 1))) ++q;
  int e = sh - k;  // value = q * 2^e
  if (q == (uint64_t(1) << 24)) {
    q >>= 1;
    ++e;
  }
  const uint32_t bits = (uint32_t(e + 23 + 127) << 23) | uint32_t(q - (uint64_t(1) << 23));
  return __builtin_bit_cast(float, bits);
}

struct Mag8 {
  float v[128];
};

constexpr Mag8 make_fp8_magnitudes() {
  Mag8 t{};
  t.v[0] = 0.0f;
  for (int i = 1; i < 128; ++i) {
    const int e = i >> 3, m = i & 7;
    // (e == 0 ? m / 8 * 2^-6 : (1 + m / 8) * 2^(e - 7)) / 480
    const uint64_t mant = e == 0 ? uint64_t(m) : uint64_t(8 + m);
    const int sh = e == 0 ? -9 : e - 10;
    t.v[i] = f32_of_ratio(mant, sh, 480);
  }
  return t;
}

constexpr Mag8 make_int8_magnitudes() {
  Mag8 t{};
  t.v[0] = 0.0f;
  int i = 1;
  for (int z = 6; z >= 0; --z) {
    const int n = 6 - z;
    uint64_t p10 = 1;
    for (int j = 0; j <= z; ++j) p10 *= 10;  // 10^(z + 1)
    for (int f = 0; f < (1 << n); ++f) {
      // 10^-z (0.1 + 0.9 (f + 1) / 2^n) = (2^n + 9 (f + 1)) / (10^(z + 1) 2^n)
      t.v[i++] = f32_of_ratio(uint64_t(1 << n) + 9 * uint64_t(f + 1), -n, p10);
    }
  }
  return t;
}

// indexed by the codebook (E4B_CB_INT8 - 4, E4B_CB_FP8 - 4)
static constexpr Mag8 kMag8[2] = {make_int8_magnitudes(), make_fp8_magnitudes()};

static_assert(kMag8[0].v[127] == 1.0f && kMag8[1].v[127] == 1.0f, "the top magnitude is 1");
static_assert(kMag8[1].v[126] == 448.0f / 480.0f, "E4M3 448 / 480");

}  // namespace e4b
