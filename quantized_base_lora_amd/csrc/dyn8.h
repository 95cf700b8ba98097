// The 8-bit dynamic tree type of the block-wise quantized optimizer states
// (Dettmers et al., "8-bit Optimizers via Block-wise Quantization", block-wise
// quantization and dynamic tree quantization): a code's magnitude bits are z
// zero bits, a one bit, then f bits holding q, standing for
// 10^-z * (0.1 + 0.9 (q + 1) / 2^f) (the 2^f fraction levels evenly in
// (0.1, 1], the top one at 1); all-zero bits stand for 0.  The signed type
// (first moment) has a sign bit and 7 magnitude bits, the unsigned type
// (second moment) 8 magnitude bits.  Read as an unsigned integer the
// magnitude bits order the values, so a code is the rank of its level.
// Levels are computed in double and rounded once to float; the decision
// threshold between consecutive levels is fl32(fl32(l_i + l_i+1) * 0.5).
// Built at compile time, for the device tables and the host query alike.
#pragma once

namespace ql {

constexpr int kAdamw8Block = 2048;   // elements per block-wise scale

struct Dyn8Table {
  float level[256];
  float thresh[255];
  int count;                          // 128 (signed magnitudes) or 256
};

constexpr Dyn8Table make_dyn8(bool is_signed) {
  Dyn8Table t{};
  const int bits = is_signed ? 7 : 8;
  t.count = 1 << bits;
  t.level[0] = 0.0f;
  for (int code = 1; code < t.count; ++code) {
    int width = 0;                    // position of the leading one bit, plus one
    for (int v = code; v; v >>= 1) ++width;
    const int z = bits - width, f = bits - 1 - z;
    const int q = code & ((1 << f) - 1);
    double p10 = 1.0;
    for (int i = 0; i < z; ++i) p10 *= 10.0;
    t.level[code] = (float)((0.1 + 0.9 * (q + 1) / (double)(1 << f)) / p10);
  }
  for (int i = 0; i + 1 < t.count; ++i) t.thresh[i] = (float)(t.level[i] + t.level[i + 1]) * 0.5f;
  return t;
}

}  // namespace ql
