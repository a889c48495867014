// Scalar-quantization helpers shared by the quantize kernels: the Lloyd-Max
// cell search over a codebook's thresholds and the LSB-first packing of 32
// codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Thresholds of one codebook held in registers (copied once from the kernel
// arguments, so the selects below are register selects, not memory loads).
template <int BITS>
struct Thresholds {
  float t[(1 << BITS) - 1];
  bool sym;   // t[L-2-k] == -t[k] and the middle one is 0
};

// Symmetric codebook: the search on |z| over the positive half.
template <int BITS>
__device__ inline int encode_sym(float z, const Thresholds<BITS>& th) {
  constexpr int half = 1 << (BITS - 1);
  const float* p = th.t + half;   // positive thresholds
  const float x = fabsf(z);
  int n;
  if constexpr (BITS == 1) {
    n = 0;
  } else if constexpr (BITS == 2) {
    n = x >= p[0];
  } else if constexpr (BITS == 3) {
    const bool b1 = x >= p[1];
    const bool b0 = x >= (b1 ? p[2] : p[0]);
    n = (b1 << 1) | b0;
  } else {
    const bool b2 = x >= p[3];
    const bool b1 = x >= (b2 ? p[5] : p[1]);
    const float tc = b2 ? (b1 ? p[6] : p[4]) : (b1 ? p[2] : p[0]);
    const bool b0 = x >= tc;
    n = (b2 << 2) | (b1 << 1) | b0;
  }
  return (half + n) ^ (z < 0.f ? 2 * half - 1 : 0);
}

// Any ascending thresholds: branch-free binary search.
template <int BITS>
__device__ inline int encode_any(float z, const Thresholds<BITS>& th) {
  const float* t = th.t;
  if constexpr (BITS == 1) {
    return z >= t[0];
  } else if constexpr (BITS == 2) {
    const bool b1 = z >= t[1];
    const bool b0 = z >= (b1 ? t[2] : t[0]);
    return (b1 << 1) | b0;
  } else if constexpr (BITS == 3) {
    const bool b2 = z >= t[3];
    const bool b1 = z >= (b2 ? t[5] : t[1]);
    const float tc = b2 ? (b1 ? t[6] : t[4]) : (b1 ? t[2] : t[0]);
    const bool b0 = z >= tc;
    return (b2 << 2) | (b1 << 1) | b0;
  } else {
    const bool b3 = z >= t[7];
    const bool b2 = z >= (b3 ? t[11] : t[3]);
    const float t1 = b3 ? (b2 ? t[13] : t[9]) : (b2 ? t[5] : t[1]);
    const bool b1 = z >= t1;
    const float t0 = b3 ? (b2 ? (b1 ? t[14] : t[12]) : (b1 ? t[10] : t[8]))
                        : (b2 ? (b1 ? t[6] : t[4]) : (b1 ? t[2] : t[0]));
    const bool b0 = z >= t0;
    return (b3 << 3) | (b2 << 2) | (b1 << 1) | b0;
  }
}

// Lloyd-Max cell index: number of thresholds t_i (ascending) with z >= t_i.
// For a codebook that mirrors around 0 (the canonical one), the search runs on
// |z| over the positive half and a negative z takes the mirrored cell
// (2^bits - 1 - cell of |z|); an exact tie with a threshold may then land in
// the neighbouring cell, which is the decision boundary itself. Otherwise a
// branch-free binary search over all thresholds. SYM = 1 or 0 fixes the case
// at compile time (the caller tested th.sym once for many codes); -1 tests it.
template <int BITS, int SYM = -1>
__device__ inline int encode(float z, const Thresholds<BITS>& th) {
  if constexpr (SYM == 1) return encode_sym<BITS>(z, th);
  else if constexpr (SYM == 0) return encode_any<BITS>(z, th);
  else return th.sym ? encode_sym<BITS>(z, th) : encode_any<BITS>(z, th);
}

// Pack 32 codes (bytes of q[0..7], LSB first) into BITS words, stream position BITS*k.
template <int BITS>
__device__ inline void pack32(const uint32_t* q, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = 0u;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t code = (q[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    const int pos = BITS * k;
    const int wi = pos >> 5, off = pos & 31;
    w[wi] |= code << off;
    if (off + BITS > 32) w[wi + 1] |= code >> (32 - off);
  }
}

}  // namespace tq
