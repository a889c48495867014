// Device helpers for gfx950 (CDNA4): bounds-checked buffer loads, MFMA operand
// types, cross-lane moves, compile-time bit-field extraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// instead of touching memory (word 3 = 0x00020000 is the gfx9-family raw format).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ inline u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ inline u32x3 bload96(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0);
}
__device__ inline u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Reinterpret a dword as float. Use this (not __builtin_bit_cast) on vector
// elements: a bit_cast of an ext_vector element expression reads element 0.
__device__ inline float as_float(uint32_t u) { return __uint_as_float(u); }

// Load N consecutive dwords at byte offset `off` (N = 1..8) into w[].
template <int N>
__device__ inline void bload_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* w) {
  if constexpr (N == 1) {
    w[0] = bload32(r, off);
  } else if constexpr (N == 2) {
    u32x2 v = bload64(r, off); w[0] = v.x; w[1] = v.y;
  } else if constexpr (N == 3) {
    u32x3 v = bload96(r, off); w[0] = v.x; w[1] = v.y; w[2] = v.z;
  } else if constexpr (N == 4) {
    u32x4 v = bload128(r, off); w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else if constexpr (N == 6) {
    u32x3 a = bload96(r, off), b = bload96(r, off + 12);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = b.x; w[4] = b.y; w[5] = b.z;
  } else if constexpr (N == 8) {
    u32x4 a = bload128(r, off), b = bload128(r, off + 16);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
    static_assert(N == 1, "unsupported word count");
  }
}

// Bits [POS, POS+W) of the LSB-first stream held in w[] (W <= 32, POS compile-time).
template <int POS, int W>
__device__ inline uint32_t field(const uint32_t* w) {
  constexpr int wi = POS / 32, off = POS % 32;
  if constexpr (off + W <= 32) {
    if constexpr (W == 32) return w[wi];
    else return __builtin_amdgcn_ubfe(w[wi], off, W);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & ((1u << W) - 1u);
  }
}

// Value from lane (lane ^ 8) inside each 16-lane row (DPP row rotate by 8).
__device__ inline float dpp_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

__device__ inline float shfl_xor_f(float x, int m) { return __shfl_xor(x, m); }

// DPP lane exchanges inside a 16-lane row: the values of lanes lane ^ 1 and
// lane ^ 2 (quad permutes) and of lane (lane - 4) mod 16 (row rotate right).
__device__ inline float dpp_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ inline float dpp_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}
__device__ inline float dpp_ror4(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
}

// Value of lane 4 * (lane / 4) + R: DPP quad permute [R, R, R, R] (R known
// after loop unrolling; the switch folds away). A multiply that consumes it
// takes the permute as its DPP source operand.
__device__ inline float quad_bcast(float x, int r) {
  const int v = __builtin_bit_cast(int, x);
  switch (r) {
    case 0: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x00, 0xF, 0xF, false));
    case 1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x55, 0xF, 0xF, false));
    case 2: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xAA, 0xF, 0xF, false));
    default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xFF, 0xF, 0xF, false));
  }
}

// Value of lane 16 * (lane / 16) + N: DPP row_newbcast (gfx90a and later).
template <int N>
__device__ inline float bcast_row_c(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}
// The same broadcast as a plain DPP move (no old value to preserve: every lane
// reads a valid lane), for a value that several instructions use.
template <int N>
__device__ inline float bcast_row_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, true));
}

// Same with n known only after loop unrolling (the switch folds away).
__device__ inline float bcast_row(float x, int n) {
  switch (n) {
    case 0: return bcast_row_c<0>(x);
    case 1: return bcast_row_c<1>(x);
    case 2: return bcast_row_c<2>(x);
    case 3: return bcast_row_c<3>(x);
    case 4: return bcast_row_c<4>(x);
    case 5: return bcast_row_c<5>(x);
    case 6: return bcast_row_c<6>(x);
    default: return bcast_row_c<7>(x);
  }
}

__device__ inline uint32_t pack_half2(float lo, float hi) {
  half2v h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ inline half8 words_to_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ inline floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace tq
