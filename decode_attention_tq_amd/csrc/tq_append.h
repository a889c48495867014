// Single-token append (quantize step of the ai-accelerate.xyz TurboQuant
// article, section "TurboQuantの仕組み", step 1), in phases that the caller
// orders with workgroup barriers between them; used by the append kernels and
// by the decode kernel when it takes the new token itself:
//   loads   the row segments of Pi (tq_rotate.h), the vector (threads 0-31),
//           a value block's words (threads 0-31 of the finishing wavefront),
//           issued early and in flight meanwhile;
//   begin   the power-of-two scale and norm, the scaled vector and
//           sqrt(d)/|x| into LDS;
//   rotate  y = Pi x in float32 FMAs (rotate_rows, one vector);
//   encode  z = y * sqrt(d)/|x| and the Lloyd-Max cell of each coordinate
//           into LDS (threads 0-127);
//   finish  the norm and the codes packed and stored (a value block keeps the
//           bits of its other tokens); keys need threads 0-3, values 0-31 of
//           the wavefront that loaded the block's words.
#pragma once

#include <math.h>
#include <stdint.h>

#include "tq_codec.h"
#include "tq_internal.h"
#include "tq_rotate.h"

namespace tq {

struct QuantArgs {
  const void* x;
  int64_t sb, st, sh;          // element strides of x
  int64_t B, T, H_kv, T_cap;
  int64_t t_offset, t_base;    // t_base = floor8(t_offset)
  int64_t nslot;               // slots per head (multiple of 8)
  int64_t n_tiles;
  uint32_t* codes;
  float* norms;
  uint32_t* signs;
  float* gamma;
  const float* rot;
  const float* proj;
  float cent[16];
  float thr[16];
  int thr_sym;   // the thresholds mirror around 0 (middle one is 0)
  PageMap pm;    // block table of a paged cache (pm.table == nullptr: contiguous)
};

// Arguments of quantizing x [B][T][H_kv][d] (element strides sb, st, sh) into
// dst at token t_offset (host; defined with the quantize kernels).
QuantArgs make_quant_args(const void* x, int64_t B, int64_t T, int64_t H_kv, int64_t sb, int64_t st, int64_t sh,
                          const tq_cache* dst, int64_t t_offset);

// Token row of (row*H_kv + head, token) in a cache's arrays: contiguous, or
// through the block table. -1 when the table maps the token's block outside
// the arrays (such a write is skipped: the table is the caller's).
__device__ inline int64_t tok_row(const PageMap& pm, int64_t H_kv, int64_t T_cap, int64_t bh, int64_t t) {
  if (pm.table == nullptr) return bh * T_cap + t;
  const uint32_t hk = (uint32_t)H_kv;
  const uint32_t b = (uint32_t)bh / hk, h = (uint32_t)bh - b * hk;   // B, H_kv < 2^16
  const int64_t blk = t >> pm.lg;
  if (blk < 0 || blk >= pm.maxblk) return -1;
  const int32_t p = pm.table[(int64_t)b * pm.maxblk + blk];
  if (p < 0 || p >= pm.nblk) return -1;
  return (((int64_t)p * H_kv + h) << pm.lg) + (t & ((int64_t(1) << pm.lg) - 1));
}

template <int BITS>
__device__ inline Thresholds<BITS> load_thresholds(const QuantArgs& a) {
  Thresholds<BITS> th;
#pragma unroll
  for (int i = 0; i < (1 << BITS) - 1; ++i) th.t[i] = a.thr[i];
  th.sym = a.thr_sym != 0;
  return th;
}

// One vector gv = row*H_kv + head at token t (LDS: xs and ys 128 floats each,
// fz 2 floats (sqrt(d)/|x| and |x|), cb 128 bytes); lt numbers the threads
// of each phase from 0.
template <int BITS, int ROLE>
struct AppendOne {
  static constexpr int KW = 4 * BITS;     // words per key token
  static constexpr int VBW = 32 * BITS;   // words per value block
  uint32_t old_words[ROLE == TQ_VALUES ? BITS : 1];
  uint32_t* vdst = nullptr;

  // values: thread cg < 32 rewrites BITS words of the block record
  // (coordinates 4cg .. 4cg+3 of the block's 8 tokens) in finish
  __device__ void load_old(const QuantArgs& a, int64_t gv, int64_t t, int lt) {
    if constexpr (ROLE == TQ_VALUES) {
      const int64_t row = lt < 32 ? tok_row(a.pm, a.H_kv, a.T_cap, gv, t & ~(int64_t)7) : -1;
      if (row >= 0) {
        vdst = a.codes + row * (VBW / 8) + (lt & 31) * BITS;
#pragma unroll
        for (int k = 0; k < BITS; ++k) old_words[k] = vdst[k];
      }
    }
  }

  // thread c4 < 32: coordinates 4c4 .. 4c4+3 of the vector (others: zeros)
  __device__ static void load_x(const QuantArgs& a, int64_t gv, int lt, bool xf32, float (&x)[4]) {
    x[0] = x[1] = x[2] = x[3] = 0.f;
    if (lt < 32) {
      const int64_t b = gv / a.H_kv, h = gv % a.H_kv;
      const int64_t off = b * a.sb + h * a.sh + 4 * (lt & 31);
      if (xf32) {
        const float4 f = *(const float4*)((const float*)a.x + off);
        x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
      } else {
        const uint2 u = *(const uint2*)((const uint16_t*)a.x + off);
        x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xFFFF0000u);
        x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xFFFF0000u);
      }
    }
  }

  // (the other threads of the 32-lane group only join the shuffles)
  __device__ void begin(const QuantArgs& a, int64_t gv, int64_t t, int lt, float (&x)[4], float* xs, float* fz) {
    const int c4 = lt & 31;
    const bool act = lt < 32;
    float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    const int sexp = (mx > 0.f) ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = ldexpf(x[u], sexp);
      ss = fmaf(x[u], x[u], ss);
    }
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m);
    const float ns = sqrtf(ss);   // |x| * 2^sexp
    if (act) *(float4*)&xs[4 * c4] = make_float4(x[0], x[1], x[2], x[3]);
    if (lt == 0) {
      fz[0] = ns > 0.f ? sqrtf((float)kD) / ns : 0.f;
      fz[1] = ldexpf(ns, -sexp);
    }
  }

  // coordinate i < 128: its Lloyd-Max cell from y_i (ys = Pi x of the scaled vector)
  __device__ static void encode_coord(const Thresholds<BITS>& th, int i, const float* ys, const float* fz,
                                      unsigned char* cb) {
    cb[i] = (unsigned char)encode<BITS>(ys[i] * *fz, th);
  }

  __device__ void finish(const QuantArgs& a, int64_t gv, int64_t t, int lt, const float* fz,
                         const unsigned char* cb) {
    if (lt == 0) {
      const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, gv, t);
      if (row >= 0) a.norms[row] = fz[1];
    }
    if constexpr (ROLE == TQ_KEYS) {
      if (lt < 4) {
        const int grp = lt;
        const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, gv, t);
        if (row >= 0) {
          uint32_t q[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) q[k] = *(const uint32_t*)&cb[32 * grp + 4 * k];
          uint32_t w[BITS];
          pack32<BITS>(q, w);
          uint32_t* dst = a.codes + row * KW + grp * BITS;
#pragma unroll
          for (int k = 0; k < BITS; ++k) dst[k] = w[k];
        }
      }
    } else {
      // thread cg: the BITS words of the block record that hold coordinates
      // 4cg .. 4cg+3 of all 8 tokens; only the new token's bits change
      if (vdst != nullptr) {
        const int cg = lt & 31;
        const int ti = (int)(t & 7);
        uint32_t w[BITS], clr[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
          w[k] = 0u;
          clr[k] = 0u;
        }
        const uint32_t q4 = *(const uint32_t*)&cb[4 * cg];
        constexpr uint32_t fm = (1u << BITS) - 1u;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t code = (q4 >> (8 * jj)) & 0xFFu;
          const int pos = BITS * (8 * jj + ti);
          const int wi = pos >> 5, off = pos & 31;
          w[wi] |= code << off;
          clr[wi] |= fm << off;
          if (off + BITS > 32) {
            w[wi + 1] |= code >> (32 - off);
            clr[wi + 1] |= fm >> (32 - off);
          }
        }
#pragma unroll
        for (int k = 0; k < BITS; ++k) vdst[k] = (old_words[k] & ~clr[k]) | w[k];
      }
    }
  }
};

}  // namespace tq
