// tables.h -- moduli, CRT weights and scaling constants, built on the host
// once per number of moduli ([Q] section 256以下の法の選び方(手順2): the
// moduli and the weights are computed ahead of time and kept in a table).
#pragma once

#include <stdint.h>

#include "common.h"

namespace oz2 {

struct Tables {
    int n = 0;
    int32_t moduli[kMaxModuli] = {};
    uint32_t weight[kMaxModuli][8] = {};  // W_l, little-endian 32-bit limbs
    int weight_limbs = 0;
    double Pp = 0.0;                      // P'_prop, rounded down
    SplitConsts split{};
    CrtConsts crt{};
    ModConsts mod{};
    CheckConsts check{};  // against modulus n + 1 (n < kMaxModuli only)
};

// Fills out[0..n) with the n largest pairwise-coprime integers <= 256 taken
// greedily from 256 downward. Returns false if n is out of range.
bool greedy_moduli(int n, int32_t *out);

// Tables for n moduli, 2 <= n <= kMaxModuli; built on first use, then cached
// (thread-safe). Returns nullptr for n out of range.
const Tables *get_tables(int n);

}  // namespace oz2
