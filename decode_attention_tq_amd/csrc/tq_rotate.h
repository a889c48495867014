// Rotation of a few float32 vectors by a 128 x 128 matrix whose rows are read
// straight from memory in segments: the query rotation of the decode prologue
// and the one-token append (the same arithmetic in both, so that an append
// fused into a decode writes the codes a separate append would).
#pragma once

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

// q' = M q for the G query heads of a workgroup: out[h][i] = sum_j M[i][j]
// in[h][j] (in, out: LDS [G][d]). Thread t takes rows R*(t/16) .. R*(t/16)+R-1
// of M (R = 2048 / NT) over the 8 columns 8*(t%16) .. 8*(t%16)+7, loaded
// straight from memory (16 consecutive lanes read whole rows; each element of
// M is read once, no staging), so every query element read from LDS serves R
// rows. The 16 segments of a row group sit in the 16 lanes of a DPP row and
// are summed with DPP exchanges, for all heads at once.
template <int NT>
struct RowSegment {
  static constexpr int R = 16 * kD / NT;   // rows per thread
  float4 r[2 * R];                        // row k: r[2k], r[2k + 1]
};

template <int NT>
__device__ inline void load_row_segment(RowSegment<NT>& rs, const float* M) {
  constexpr int R = RowSegment<NT>::R;
  const int i0 = R * (threadIdx.x / 16), sg = threadIdx.x % 16;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    rs.r[2 * k] = *(const float4*)(M + (i0 + k) * kD + 8 * sg);
    rs.r[2 * k + 1] = *(const float4*)(M + (i0 + k) * kD + 8 * sg + 4);
  }
}

template <int NT, int MAXG>
__device__ inline void rotate_rows(const RowSegment<NT>& rs, const float* in, float* out, int G) {
  constexpr int R = RowSegment<NT>::R;
  const int i0 = R * (threadIdx.x / 16), sg = threadIdx.x % 16;
  float acc[MAXG][R];
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
#pragma unroll
    for (int k = 0; k < R; ++k) acc[h][k] = 0.f;
    if (h < G) {
      const float4 a = *(const float4*)(in + h * kD + 8 * sg);
      const float4 b = *(const float4*)(in + h * kD + 8 * sg + 4);
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const float4 m0 = rs.r[2 * k], m1 = rs.r[2 * k + 1];
        const float v = fmaf(m0.x, a.x, fmaf(m0.y, a.y, fmaf(m0.z, a.z, m0.w * a.w)));
        acc[h][k] = fmaf(m1.x, b.x, fmaf(m1.y, b.y, fmaf(m1.z, b.z, fmaf(m1.w, b.w, v))));
      }
    }
  }
  // sums over the 16 lanes of the row: quads, then rotates by 4 and 8 (every
  // lane ends with the full sum)
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float v = acc[h][k] + dpp_xor1(acc[h][k]);
      v += dpp_xor2(v);
      v += dpp_ror4(v);
      v += dpp_ror8(v);
      acc[h][k] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < MAXG; ++h) {
    if (h < G && sg == h) {
#pragma unroll
      for (int k = 0; k < R; ++k) out[h * kD + i0 + k] = acc[h][k];
    }
  }
}

}  // namespace tq
