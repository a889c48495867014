// Quantize and dequantize kernels for the packed TurboQuant cache, for gfx950.
//
// quantize (ai-accelerate.xyz TurboQuant article, section "TurboQuantの仕組み",
// step 1, and step 2 for QJL keys), per vector x:
//   n = |x|; y = Pi x on MFMA; z = y * sqrt(d) / n (the rotated unit vector in
//   standard-normal units); code_j = #{ i : z_j >= t_i } for the Lloyd-Max
//   thresholds t; codes are bit-packed into the key or value layout; n is stored.
//   QJL keys: rho = z - c[code]; gamma = |rho| / sqrt(d); sign bits of S rho.
//
// Rotation precision: the input is scaled per vector by a power of two so its
// largest entry lies in [2^13, 2^14) and converted to float16, which is exact for
// bfloat16 input (8 significant bits) above float16's normal range floor;
// float32 input is split into float16 hi + lo. Pi (and S) are split into float16
// hi + lo once per workgroup, so the MFMA products carry ~22 significant bits and
// the float32 accumulation gives y to ~1e-7 relative, far inside the 1e-6
// decision-boundary band.
//
// Work decomposition: "slots" enumerate, per (row, head), the token range
// [floor8(t_offset), ceil8(t_offset + T)); a tile is 16 or 32 slots per
// wavefront, so a tile always holds whole 8-token value blocks and short
// appends (T = 1) of many heads share one workgroup. Workgroups are
// persistent: each loads Pi once into LDS (in MFMA operand order) and loops
// over tiles, with the next tile's input in flight. Bulk quantization without
// QJL uses 32-slot tiles on 32x32x16 MFMAs (16 wavefronts per workgroup);
// short inputs and QJL keys use 16-slot tiles on 16x16x32 MFMAs; a single
// token per (row, head) without QJL takes the append kernel (float32 FMAs).
#include <math.h>

#include <atomic>

#include "tq_append.h"
#include "tq_codec.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {

namespace {

// (row * H_kv + head, token) of slot s0 + v, for a wave-uniform first slot s0
// of a wavefront's tile and a small lane offset v: the 64-bit division runs
// once on the scalar unit, each lane does a 32-bit one (nslot < 2^31).
__device__ inline void slot_pos(const QuantArgs& a, int64_t s0, uint32_t v, int64_t& bh, int64_t& t) {
  const int64_t bh0 = s0 / a.nslot;
  const uint32_t ns = (uint32_t)a.nslot;
  const uint32_t rr = (uint32_t)(s0 - bh0 * a.nslot) + v;
  const uint32_t q = rr / ns;
  bh = bh0 + q;
  t = a.t_base + (int64_t)(rr - q * ns);
}


// Load Pi (or S), split into float16 hi/lo, into LDS in B-operand order:
// op[pass][ks][nb][lane][8] = M[16nb + n][32g + 8ks + e], lane = 16g + n.
// Every thread issues all of its 16-byte loads before converting, so the
// matrix arrives in about one memory latency.
template <int NT>
__device__ void stage_matrix(const float* M, _Float16* op) {
  constexpr int PER = kD * kD / 4 / NT;
  float4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = ((const float4*)M)[threadIdx.x + k * NT];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = 4 * (threadIdx.x + k * NT);
    const int row = idx / kD, col = idx % kD;
    const int nb = row >> 4, n = row & 15;
    const int g = col >> 5, ks = (col >> 3) & 3, e = col & 7;   // e is 0 or 4
    const int o = (((ks * 8 + nb) * 64 + 16 * g + n) << 3) + e;
    const float x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    _Float16 hi[4], lo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hi[u] = (_Float16)x[u];
      lo[u] = (_Float16)(x[u] - (float)hi[u]);
    }
    *(uint2*)(op + o) = make_uint2(pack_half2((float)hi[0], (float)hi[1]), pack_half2((float)hi[2], (float)hi[3]));
    *(uint2*)(op + 4 * 8 * 64 * 8 + o) =
        make_uint2(pack_half2((float)lo[0], (float)lo[1]), pack_half2((float)lo[2], (float)lo[3]));
  }
}

// Wavefronts per quantize workgroup. Without QJL a workgroup of 8 shares one
// copy of Pi (64 KB) and two fit a compute unit (16 wavefronts); the QJL
// variant also holds S and its residual buffers.
template <int QJL>
constexpr int quant_waves() { return QJL ? 2 : 8; }

// Wave-local exchange through LDS: the lanes of one wavefront write, then read
// what other lanes wrote. LDS operations of a wavefront complete in order, so
// this only has to keep the compiler from moving memory operations across it.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raw input of one slot-row of a tile: the lane's 32 coordinates, as loaded.
template <int XF32>
struct RawX {
  u32x4 v[XF32 ? 8 : 4];
  bool valid;
};

template <int WAVES, int XF32>
__device__ inline void load_raw(RawX<XF32>& r, const QuantArgs& a, int64_t tile, int wave, int g, int i16) {
  constexpr int TILE = 16 * WAVES;
  int64_t bh, t;
  slot_pos(a, tile * TILE + wave * 16, i16, bh, t);
  r.valid = bh < a.B * a.H_kv && t >= a.t_offset && t < a.t_offset + a.T;
  if (r.valid) {
    const int64_t b = bh / a.H_kv, h = bh % a.H_kv;
    const int64_t off = b * a.sb + (t - a.t_offset) * a.st + h * a.sh + 32 * g;
    const u32x4* p = XF32 ? (const u32x4*)((const float*)a.x + off) : (const u32x4*)((const uint16_t*)a.x + off);
#pragma unroll
    for (int k = 0; k < (XF32 ? 8 : 4); ++k) r.v[k] = p[k];
  } else {
#pragma unroll
    for (int k = 0; k < (XF32 ? 8 : 4); ++k) r.v[k] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int BITS, int ROLE, int QJL, int XF32>
__global__ __launch_bounds__(64 * quant_waves<QJL>()) void quantize_kernel(QuantArgs a) {
  constexpr int WAVES = quant_waves<QJL>();
  const Thresholds<BITS> th = load_thresholds<BITS>(a);
  constexpr int NT = 64 * WAVES;
  constexpr int TILE = 16 * WAVES;
  constexpr int OPH = 4 * 8 * 64 * 8;   // halves per pass of an operand matrix
  constexpr int KW = 4 * BITS;          // words per key token
  constexpr int VBW = 32 * BITS;        // words per value block
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* piop = (_Float16*)smem;                                  // 2 * OPH halves
  _Float16* sop = piop + 2 * OPH;                                   // QJL: 2 * OPH halves
  unsigned char* cbuf_all = (unsigned char*)(piop + (QJL ? 4 : 2) * OPH);   // WAVES * 16 * 128 bytes
  _Float16* rbuf_all = (_Float16*)(cbuf_all + WAVES * 16 * kD);       // QJL: WAVES * 2 * 16 * 128 halves

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  // the first tile's input is in flight while Pi is staged
  RawX<XF32> cur;
  if (blockIdx.x < a.n_tiles) load_raw<WAVES, XF32>(cur, a, blockIdx.x, wave, g, i16);
  stage_matrix<NT>(a.rot, piop);
  if constexpr (QJL) stage_matrix<NT>(a.proj, sop);
  __syncthreads();

  unsigned char* cbuf = cbuf_all + wave * 16 * kD;
  _Float16* rhi = rbuf_all + wave * 2 * 16 * kD;
  _Float16* rlo = rhi + 16 * kD;
  const float sqrt_d = sqrtf((float)kD);
  const int64_t heads = a.B * a.H_kv;

  // the input of the next tile is loaded while the current one is processed
  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    RawX<XF32> nxt;
    if (tile + gridDim.x < a.n_tiles) load_raw<WAVES, XF32>(nxt, a, tile + gridDim.x, wave, g, i16);
    // ---- slot of this lane (row i16 of the wave's 16)
    int64_t bh, t;
    slot_pos(a, tile * TILE + wave * 16, i16, bh, t);
    const bool valid = cur.valid;

    // ---- the lane's 32 coordinates (32g .. 32g+31) as float32
    float xv[32];
    if constexpr (XF32) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[4 * k + u] = __uint_as_float(cur.v[k][u]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xv[8 * k + 2 * u] = __uint_as_float(cur.v[k][u] << 16);
          xv[8 * k + 2 * u + 1] = __uint_as_float(cur.v[k][u] & 0xFFFF0000u);
        }
      }
    }

    // ---- power-of-two scale, norm
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) mx = fmaxf(mx, fabsf(xv[k]));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const int sexp = (mx > 0.f) ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      xv[k] = ldexpf(xv[k], sexp);
      ss = fmaf(xv[k], xv[k], ss);
    }
    ss += shfl_xor_f(ss, 16);
    ss += shfl_xor_f(ss, 32);
    const float ns = sqrtf(ss);                      // |x| * 2^sexp
    const float fz = ns > 0.f ? sqrt_d / ns : 0.f;   // z = y_scaled * fz

    // ---- A operand (x as float16 hi/lo), coordinates 32g + 8ks + e
    half8 xa[4], xl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = xv[8 * ks + e];
        const _Float16 hi = (_Float16)v;
        xa[ks][e] = hi;
        if constexpr (XF32) xl[ks][e] = (_Float16)(v - (float)hi);
      }
    }

    // ---- y = Pi x on MFMA: D[nb] lane (g, n) = y[slot 4g + r][16nb + n]
    floatx4 y[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      floatx4 accv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int o = ((ks * 8 + nb) * 64 + lane) << 3;
        const half8 bh8 = *(const half8*)(piop + o);
        const half8 bl8 = *(const half8*)(piop + OPH + o);
        accv = mfma16(xa[ks], bh8, accv);
        accv = mfma16(xa[ks], bl8, accv);
        if constexpr (XF32) accv = mfma16(xl[ks], bh8, accv);
      }
      y[nb] = accv;
    }

    // ---- codes
    float fr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) fr[r] = __shfl(fz, 4 * g + r);
    int code[8][4];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float z = y[nb][r] * fr[r];
        y[nb][r] = z;
        code[nb][r] = encode<BITS>(z, th);
        cbuf[(4 * g + r) * kD + 16 * nb + i16] = (unsigned char)code[nb][r];
      }
    }

    // ---- QJL residual sketch (keys)
    float gam[4];
    if constexpr (QJL) {
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float cc = a.cent[0];
#pragma unroll
          for (int q = 1; q < (1 << BITS); ++q) cc = (code[nb][r] == q) ? a.cent[q] : cc;
          const float rho = y[nb][r] - cc;
          rs[r] = fmaf(rho, rho, rs[r]);
          const _Float16 hi = (_Float16)rho;
          rhi[(4 * g + r) * kD + 16 * nb + i16] = hi;
          rlo[(4 * g + r) * kD + 16 * nb + i16] = (_Float16)(rho - (float)hi);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) rs[r] += shfl_xor_f(rs[r], m);
        gam[r] = sqrtf(rs[r]) / sqrt_d;
      }
    }
    wave_sync();

    if constexpr (QJL) {
      // z' = S rho on MFMA; A operand rows = slots, coordinates 32g + 8ks + e
      half8 ra[4], rl[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ra[ks] = *(const half8*)(rhi + i16 * kD + 32 * g + 8 * ks);
        rl[ks] = *(const half8*)(rlo + i16 * kD + 32 * g + 8 * ks);
      }
      wave_sync();
      unsigned char* sbuf = (unsigned char*)rhi;   // reuse: sign bytes [slot][coord]
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        floatx4 accv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int o = ((ks * 8 + nb) * 64 + lane) << 3;
          const half8 bh8 = *(const half8*)(sop + o);
          const half8 bl8 = *(const half8*)(sop + OPH + o);
          accv = mfma16(ra[ks], bh8, accv);
          accv = mfma16(ra[ks], bl8, accv);
          accv = mfma16(rl[ks], bh8, accv);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sbuf[(4 * g + r) * kD + 16 * nb + i16] = accv[r] >= 0.f ? 1 : 0;
      }
      wave_sync();
      // signs + gamma: lane (v = lane/4, grp = lane%4) packs 32 sign bits of slot v
      {
        const int v = lane >> 2, grp = lane & 3;
        int64_t bh2, t2;
        slot_pos(a, tile * TILE + wave * 16, v, bh2, t2);
        const bool ok = bh2 < heads && t2 >= a.t_offset && t2 < a.t_offset + a.T;
        const uint32_t* q = (const uint32_t*)(sbuf + v * kD + 32 * grp);
        uint32_t wbits = 0u;
#pragma unroll
        for (int k = 0; k < 32; ++k) wbits |= ((q[k >> 2] >> (8 * (k & 3))) & 1u) << k;
        const int64_t row = ok ? tok_row(a.pm, a.H_kv, a.T_cap, bh2, t2) : -1;
        if (row >= 0) a.signs[row * 4 + grp] = wbits;
      }
      // gamma: lane (g, n = 0) holds slots 4g + r
      if (i16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int64_t bh2, t2;
          slot_pos(a, tile * TILE + wave * 16, 4 * g + r, bh2, t2);
          if (bh2 < heads && t2 >= a.t_offset && t2 < a.t_offset + a.T) {
            const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh2, t2);
            if (row >= 0) a.gamma[row] = gam[r];
          }
        }
      }
    }

    // ---- norms
    if (valid && g == 0) {
      const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, t);
      if (row >= 0) a.norms[row] = ldexpf(ns, -sexp);
    }

    // ---- pack and store codes
    if constexpr (ROLE == TQ_KEYS) {
      const int v = lane >> 2, grp = lane & 3;
      int64_t bh2, t2;
      slot_pos(a, tile * TILE + wave * 16, v, bh2, t2);
      const bool ok = bh2 < heads && t2 >= a.t_offset && t2 < a.t_offset + a.T;
      uint32_t q[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) q[k] = *(const uint32_t*)(cbuf + v * kD + 32 * grp + 4 * k);
      uint32_t w[BITS];
      pack32<BITS>(q, w);
      const int64_t row = ok ? tok_row(a.pm, a.H_kv, a.T_cap, bh2, t2) : -1;
      if (row >= 0) {
        uint32_t* dst = a.codes + row * KW + grp * BITS;
#pragma unroll
        for (int k = 0; k < BITS; ++k) dst[k] = w[k];
      }
    } else {
      // lane (blk = lane/32, cg = lane%32): coordinates 4cg .. 4cg+3 of the block's 8 tokens
      const int blk = lane >> 5, cg = lane & 31;
      int64_t bh2, tb;   // the block's first slot
      slot_pos(a, tile * TILE + wave * 16, 8 * blk, bh2, tb);
      uint32_t w[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k) w[k] = 0u;
      uint32_t keep[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k) keep[k] = 0u;
      bool any_valid = false, all_valid = true;
#pragma unroll
      for (int ti = 0; ti < 8; ++ti) {
        const int64_t tt = tb + ti;
        const bool ok = bh2 < heads && tt >= a.t_offset && tt < a.t_offset + a.T;
        any_valid |= ok;
        all_valid &= ok;
        const uint32_t q4 = *(const uint32_t*)(cbuf + (8 * blk + ti) * kD + 4 * cg);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t code = (q4 >> (8 * jj)) & 0xFFu;
          const int pos = BITS * (8 * jj + ti);
          const int wi = pos >> 5, off = pos & 31;
          const uint32_t fm = (1u << BITS) - 1u;
          const uint32_t okm = ok ? ~0u : 0u;   // branch-free: positions are compile-time
          w[wi] |= (code << off) & okm;
          keep[wi] |= (fm << off) & ~okm;
          if (off + BITS > 32) {
            w[wi + 1] |= (code >> (32 - off)) & okm;
            keep[wi + 1] |= (fm >> (32 - off)) & ~okm;
          }
        }
      }
      const int64_t row = any_valid ? tok_row(a.pm, a.H_kv, a.T_cap, bh2, tb) : -1;
      if (row >= 0) {
        uint32_t* dst = a.codes + row * (VBW / 8) + cg * BITS;
#pragma unroll
        for (int k = 0; k < BITS; ++k) dst[k] = all_valid ? w[k] : ((dst[k] & keep[k]) | w[k]);
      }
    }
    wave_sync();   // the code buffer is rewritten by the next tile
    cur = nxt;
  }
}

// ------------------------------------------- quantize, 32-vector tiles --
//
// Without QJL the rotation runs on v_mfma_f32_32x32x16_f16 over 32-vector
// tiles: each B operand read from LDS (a 16 x 32 slice of Pi^T, float16 hi or
// lo) now serves 32 vectors instead of 16, which halves the LDS traffic per
// vector (the limit of the 16-vector tiles). A workgroup of 16 wavefronts
// shares one copy of Pi and fills a compute unit.
//   A[i][k]  = x of vector i (32 per wave), lane i + 32*(k/8), element k % 8;
//   B[k][j]  = Pi[j][k], lane j + 32*(k/8);
//   D[i][j]  lane j + 32*((i/4)%2), element (i%4) + 4*(i/8).
constexpr int kQ32Waves = 16;
template <int V>
struct IntTag {
  static constexpr int value = V;
};
constexpr int kQ32OpHalves = 8 * 4 * 64 * 8;   // one float16 pass of Pi in operand order
// Row stride (bytes) of a wavefront's code buffer [32 vectors][128 codes]: the
// 32 lanes that write one 4-code piece of 32 different rows hit distinct banks.
constexpr int kQ32Row = kD + 4;

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ inline floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// op[pass][ks][jb][lane][e] = Pi[32jb + lane%32][16ks + 8(lane/32) + e], hi and lo passes.
__device__ void stage_matrix32(const float* M, _Float16* op) {
  constexpr int PER = kD * kD / 4 / (64 * kQ32Waves);
  float4 v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = ((const float4*)M)[threadIdx.x + k * 64 * kQ32Waves];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = 4 * (threadIdx.x + k * 64 * kQ32Waves);
    const int row = idx / kD, col = idx % kD;   // Pi[row][col..col+3]
    const int jb = row >> 5, jl = row & 31;
    const int ks = col >> 4, kh = (col >> 3) & 1, e = col & 7;   // e is 0 or 4
    const int o = (((ks * 4 + jb) * 64 + 32 * kh + jl) << 3) + e;
    const float x[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    _Float16 hi[4], lo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hi[u] = (_Float16)x[u];
      lo[u] = (_Float16)(x[u] - (float)hi[u]);
    }
    *(uint2*)(op + o) = make_uint2(pack_half2((float)hi[0], (float)hi[1]), pack_half2((float)hi[2], (float)hi[3]));
    *(uint2*)(op + kQ32OpHalves + o) =
        make_uint2(pack_half2((float)lo[0], (float)lo[1]), pack_half2((float)lo[2], (float)lo[3]));
  }
}

// The 64 coordinates of one vector that lane (i, kh) holds: 16ks + 8kh + e.
template <int XF32>
struct RawX32 {
  u32x4 v[XF32 ? 16 : 8];
  bool valid;
};

template <int XF32>
__device__ inline void load_raw32(RawX32<XF32>& r, const QuantArgs& a, int64_t tile, int wave, int vi, int kh) {
  int64_t bh, t;
  slot_pos(a, tile * (32 * kQ32Waves) + wave * 32, vi, bh, t);
  r.valid = bh < a.B * a.H_kv && t >= a.t_offset && t < a.t_offset + a.T;
  if (r.valid) {
    const int64_t b = bh / a.H_kv, h = bh % a.H_kv;
    const int64_t off = b * a.sb + (t - a.t_offset) * a.st + h * a.sh + 8 * kh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if constexpr (XF32) {
        const u32x4* p = (const u32x4*)((const float*)a.x + off + 16 * ks);
        r.v[2 * ks] = p[0];
        r.v[2 * ks + 1] = p[1];
      } else {
        r.v[ks] = *(const u32x4*)((const uint16_t*)a.x + off + 16 * ks);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < (XF32 ? 16 : 8); ++k) r.v[k] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int BITS, int ROLE, int XF32>
__global__ __launch_bounds__(64 * kQ32Waves) void quantize32_kernel(QuantArgs a) {
  constexpr int TILE = 32 * kQ32Waves;
  const Thresholds<BITS> th = load_thresholds<BITS>(a);
  constexpr int KW = 4 * BITS;          // words per key token
  constexpr int VBW = 32 * BITS;        // words per value block
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16* piop = (_Float16*)smem;                                   // 2 passes
  unsigned char* cbuf_all = (unsigned char*)(piop + 2 * kQ32OpHalves);   // [wave][32][kQ32Row] codes

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int vi = lane & 31, kh = lane >> 5;
  // the first tile's input is in flight while Pi is staged
  RawX32<XF32> cur;
  if (blockIdx.x < a.n_tiles) load_raw32<XF32>(cur, a, blockIdx.x, wave, vi, kh);
  stage_matrix32(a.rot, piop);
  __syncthreads();

  unsigned char* cbuf = cbuf_all + wave * 32 * kQ32Row;
  const float sqrt_d = sqrtf((float)kD);
  const int64_t heads = a.B * a.H_kv;

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    // (float32 input is not prefetched: its raw tile alone takes 64 VGPRs)
    RawX32<XF32> nxt;
    if (!XF32 && tile + gridDim.x < a.n_tiles) load_raw32<XF32>(nxt, a, tile + gridDim.x, wave, vi, kh);
    int64_t bh, t;
    slot_pos(a, tile * TILE + wave * 32, vi, bh, t);

    // ---- the lane's 64 coordinates, x[16ks + 8kh + e]: power-of-two scale
    // (largest entry in [2^13, 2^14)), norm, float16 A operands (hi, and lo
    // for float32 input)
    auto coord = [&](int ks, int e) -> float {
      if constexpr (XF32) return __uint_as_float(cur.v[2 * ks + (e >> 2)][e & 3]);
      else return __uint_as_float((e & 1) ? (cur.v[ks][e >> 1] & 0xFFFF0000u) : (cur.v[ks][e >> 1] << 16));
    };
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(coord(ks, e)));
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const int sexp = (mx > 0.f) ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
    float ss = 0.f;
    half8 xa[8], xl[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ldexpf(coord(ks, e), sexp);
        ss = fmaf(v, v, ss);
        const _Float16 hi = (_Float16)v;
        xa[ks][e] = hi;
        if constexpr (XF32) xl[ks][e] = (_Float16)(v - (float)hi);
      }
    }
    ss += shfl_xor_f(ss, 32);
    const float ns = sqrtf(ss);                      // |x| * 2^sexp
    const float fz = ns > 0.f ? sqrt_d / ns : 0.f;   // z = y_scaled * fz

    // ---- y = Pi x, 32 output coordinates at a time, and the codes. With Pi
    // as the A operand and x as B, lane (vi, kh) receives coordinates
    // 32jb + 8q + 4kh + r (element 4q + r) of its own vector vi, so four
    // adjacent codes leave as one 32-bit LDS write.
    // (the codebook's symmetry is tested once per tile, so the 64 code
    // searches of a lane are straight-line code)
    auto rotate_encode = [&](auto sym) {
      constexpr int SYM = decltype(sym)::value;
#pragma unroll 1
      for (int jb = 0; jb < 4; ++jb) {
        floatx16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int o = ((ks * 4 + jb) * 64 + lane) << 3;
          const half8 bh8 = *(const half8*)(piop + o);
          const half8 bl8 = *(const half8*)(piop + kQ32OpHalves + o);
          acc = mfma32(bh8, xa[ks], acc);
          acc = mfma32(bl8, xa[ks], acc);
          if constexpr (XF32) acc = mfma32(bh8, xl[ks], acc);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t word = 0u;
#pragma unroll
          for (int r = 0; r < 4; ++r) word |= (uint32_t)encode<BITS, SYM>(acc[4 * q + r] * fz, th) << (8 * r);
          *(uint32_t*)(cbuf + vi * kQ32Row + 32 * jb + 8 * q + 4 * kh) = word;
        }
      }
    };
    if (th.sym)
      rotate_encode(IntTag<1>{});
    else
      rotate_encode(IntTag<0>{});

    // ---- norm
    if (cur.valid && kh == 0) {
      const int64_t row = tok_row(a.pm, a.H_kv, a.T_cap, bh, t);
      if (row >= 0) a.norms[row] = ldexpf(ns, -sexp);
    }
    wave_sync();

    // ---- pack and store codes, 16 vectors per pass
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if constexpr (ROLE == TQ_KEYS) {
        const int v = 16 * pass + (lane >> 2), grp = lane & 3;
        int64_t bh2, t2;
        slot_pos(a, tile * TILE + wave * 32, v, bh2, t2);
        const bool ok = bh2 < heads && t2 >= a.t_offset && t2 < a.t_offset + a.T;
        uint32_t q[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = *(const uint32_t*)(cbuf + v * kQ32Row + 32 * grp + 4 * k);
        uint32_t w[BITS];
        pack32<BITS>(q, w);
        const int64_t row = ok ? tok_row(a.pm, a.H_kv, a.T_cap, bh2, t2) : -1;
        if (row >= 0) {
          uint32_t* dst = a.codes + row * KW + grp * BITS;
#pragma unroll
          for (int k = 0; k < BITS; ++k) dst[k] = w[k];
        }
      } else {
        // lane (blk, cg): coordinates 4cg .. 4cg+3 of the 8 tokens of block 2*pass + blk
        const int blk = 2 * pass + (lane >> 5), cg = lane & 31;
        int64_t bh2, tb;   // the block's first slot
        slot_pos(a, tile * TILE + wave * 32, 8 * blk, bh2, tb);
        uint32_t w[BITS], keep[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) {
          w[k] = 0u;
          keep[k] = 0u;
        }
        bool any_valid = false, all_valid = true;
#pragma unroll
        for (int ti = 0; ti < 8; ++ti) {
          const int64_t tt = tb + ti;
          const bool ok = bh2 < heads && tt >= a.t_offset && tt < a.t_offset + a.T;
          any_valid |= ok;
          all_valid &= ok;
          const uint32_t q4 = *(const uint32_t*)(cbuf + (8 * blk + ti) * kQ32Row + 4 * cg);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t code = (q4 >> (8 * jj)) & 0xFFu;
            const int pos = BITS * (8 * jj + ti);
            const int wi = pos >> 5, off = pos & 31;
            const uint32_t fm = (1u << BITS) - 1u;
            const uint32_t okm = ok ? ~0u : 0u;   // branch-free: positions are compile-time
            w[wi] |= (code << off) & okm;
            keep[wi] |= (fm << off) & ~okm;
            if (off + BITS > 32) {
              w[wi + 1] |= (code >> (32 - off)) & okm;
              keep[wi + 1] |= (fm >> (32 - off)) & ~okm;
            }
          }
        }
        const int64_t row = any_valid ? tok_row(a.pm, a.H_kv, a.T_cap, bh2, tb) : -1;
        if (row >= 0) {
          uint32_t* dst = a.codes + row * (VBW / 8) + cg * BITS;
#pragma unroll
          for (int k = 0; k < BITS; ++k) dst[k] = all_valid ? w[k] : ((dst[k] & keep[k]) | w[k]);
        }
      }
    }
    wave_sync();   // the code buffer and the scales are rewritten by the next tile
    if constexpr (XF32) {
      if (tile + gridDim.x < a.n_tiles) load_raw32<XF32>(cur, a, tile + gridDim.x, wave, vi, kh);
    } else {
      cur = nxt;
    }
  }
}

// ---------------------------------- quantize, bfloat16 input, 32-vector tiles --
//
// bfloat16 input needs no conversion on v_mfma_f32_32x32x16_bf16: the raw
// 16-byte loads of x are the MFMA operands as they stand. Pi is split once per
// workgroup into three bfloat16 parts (hi + mid + lo hold 24 significant bits,
// float32's precision), so y = Pi x takes three MFMAs per 16 coordinates, each
// product exact, accumulated in float32. The norm comes from v_dot2_f32_bf16 on
// the same words; a vector whose squared norm leaves [2^-100, 2^100] is first
// rescaled by a power of two (exact), so neither the norm nor y under- or
// overflows.
//
// Codes leave as bits, not bytes: each comparison of the cell search yields a
// lane mask, and v_addc_co_u32 (w + w + carry) shifts one such bit per lane into
// a word. A lane pushes its codes in descending stream position, so the last
// bit pushed lands at bit 0 and the words come out in the packed layout. The
// MFMA operand roles are chosen so that what a lane holds is contiguous there:
//  - keys: A = Pi, B = x. The rows of Pi are staged in the order that gives
//    lane (vector v, half h) coordinate 64h + 16jb + e in element e of block
//    jb: 2*BITS consecutive words of token v's row per lane.
//  - values: A = x, B = Pi^T. Lane (column j, half h) receives coordinate
//    32jb + j of the vectors of slots 16h + e (the rows of x are loaded in that
//    order): for each of its two 8-token blocks, the 8*BITS bits of one
//    coordinate. The four lanes of a quad (coordinates 4cg .. 4cg+3) merge
//    their pieces into the block's BITS words of that coordinate group.
// Keys compare y with thresholds scaled per vector (t_i |x| / sqrt(d)); values,
// whose lanes hold 16 vectors each, compare z = y sqrt(d) / |x|.
constexpr int kQbWaves = 16;
constexpr int kQbPart = 8 * 4 * 64;   // 16-byte pieces of one bfloat16 part of Pi
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline floatx16 mfma32bf(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Row of Pi that operand row i (0..31) of output block jb holds.
template <int ROLE>
__device__ inline int qb_pi_row(int jb, int i) {
  if constexpr (ROLE == TQ_KEYS) return 64 * ((i >> 2) & 1) + 16 * jb + (i & 3) + 4 * (i >> 3);
  else return 32 * jb + i;
}

// Slot (within the wavefront's 32) whose vector lane row i of the x operand
// holds: keys take slot i; values the order that gives output lane half h the
// slots 16h .. 16h+15 in element order.
template <int ROLE>
__device__ inline int qb_slot(int i) {
  if constexpr (ROLE == TQ_KEYS) return i;
  else return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

__device__ inline uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// op[jb][ks][part][lane] (16 bytes) = part (0 hi, 1 mid, 2 lo) of
// Pi[qb_pi_row(jb, lane % 32)][16ks + 8(lane / 32) + e]: the 24 pieces of one
// output block lie within 24 KB, so one address register and the instruction's
// immediate offset reach every read of two blocks.
__device__ inline int qb_piece(int jb, int ks, int part) { return ((jb * 8 + ks) * 3 + part) * 64; }

// A rotation whose entries all have one magnitude c (a randomized Hadamard
// matrix H diag(s) / sqrt(d)) is c times a sign matrix S, and S x is exact in a
// single bfloat16 MFMA pass: only part 0, holding the signs (+-1), is staged,
// and the caller scales y = c (S x). Otherwise the three parts of Pi. Returns
// c for a sign matrix, 0 otherwise (the same in every thread).
template <int ROLE>
__device__ float stage_matrix_bf16(const float* M, u32x4* op) {
  constexpr int NT = 64 * kQbWaves;
  constexpr int PER = kQbPart / NT;
  float4 v[PER][2];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int piece = threadIdx.x + k * NT;
    const int ln = piece & 63, ks = (piece >> 6) & 7, jb = piece >> 9;
    const float4* src = (const float4*)(M + qb_pi_row<ROLE>(jb, ln & 31) * kD + 16 * ks + 8 * (ln >> 5));
    v[k][0] = src[0];
    v[k][1] = src[1];
  }
  const float c = fabsf(M[0]);
  bool one_magnitude = c > 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    one_magnitude &= fabsf(v[k][0].x) == c && fabsf(v[k][0].y) == c && fabsf(v[k][0].z) == c &&
                     fabsf(v[k][0].w) == c && fabsf(v[k][1].x) == c && fabsf(v[k][1].y) == c &&
                     fabsf(v[k][1].z) == c && fabsf(v[k][1].w) == c;
  }
  const bool sign_matrix = __syncthreads_and(one_magnitude) != 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const float x[8] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w, v[k][1].x, v[k][1].y, v[k][1].z, v[k][1].w};
    const int piece = threadIdx.x + k * NT;
    const int ln = piece & 63, ks = (piece >> 6) & 7, jb = piece >> 9;
    if (sign_matrix) {
      uint32_t sw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sw[e] = x[e] < 0.f ? 0xBF80u : 0x3F80u;   // bfloat16 -1, +1
      op[qb_piece(jb, ks, 0) + ln] = u32x4{sw[0] | sw[1] << 16, sw[2] | sw[3] << 16, sw[4] | sw[5] << 16, sw[6] | sw[7] << 16};
      continue;
    }
    uint32_t hw[8], mw[8], lw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 hi = (__bf16)x[e];
      const float r1 = x[e] - (float)hi;
      const __bf16 mid = (__bf16)r1;
      const float r2 = r1 - (float)mid;
      hw[e] = __builtin_bit_cast(uint16_t, hi);
      mw[e] = __builtin_bit_cast(uint16_t, mid);
      lw[e] = bf16_bits(r2);
    }
    op[qb_piece(jb, ks, 0) + ln] = u32x4{hw[0] | hw[1] << 16, hw[2] | hw[3] << 16, hw[4] | hw[5] << 16, hw[6] | hw[7] << 16};
    op[qb_piece(jb, ks, 1) + ln] = u32x4{mw[0] | mw[1] << 16, mw[2] | mw[3] << 16, mw[4] | mw[5] << 16, mw[6] | mw[7] << 16};
    op[qb_piece(jb, ks, 2) + ln] = u32x4{lw[0] | lw[1] << 16, lw[2] | lw[3] << 16, lw[4] | lw[5] << 16, lw[6] | lw[7] << 16};
  }
  return sign_matrix ? c : 0.f;
}

// w * 2 + (bit of this lane in m): one code bit shifted into a word.
// The instruction is written out (the compiler folds w + w + carry into a shift
// and a select), so the compiler's hazard tracking does not see that it is a
// vector instruction reading and writing scalar registers. Two rules keep it
// safe: its carry-out goes to `sink`, a scalar pair that only these pushes
// write and that stays live across the caller's loop (a scalar instruction must
// never write a register whose vector write of lanes 32-63 may still be in
// flight), and two wait states follow it before any other instruction may
// overwrite the mask it reads.
// A mask written by a vector compare also needs two wait states before a vector
// instruction reads it: VALU_MASK = 1 puts them in front (masks made by scalar
// instructions need none).
template <int VALU_MASK>
__device__ inline uint32_t push_bit(uint32_t w, uint64_t m, uint64_t& sink) {
  uint32_t r;
  if constexpr (VALU_MASK)
    asm("s_nop 1\n\tv_addc_co_u32 %0, %1, %2, %2, %3\n\ts_nop 1" : "=v"(r), "+s"(sink) : "v"(w), "s"(m));
  else
    asm("v_addc_co_u32 %0, %1, %2, %2, %3\n\ts_nop 1" : "=v"(r), "+s"(sink) : "v"(w), "s"(m));
  return r;
}

__device__ inline uint64_t lanes(bool c) { return __builtin_amdgcn_ballot_w64(c); }

// Lane masks of the bits of code(z) (bit k in m[k]) for ascending thresholds
// t[0 .. 2^BITS - 2], the cells encode<BITS, SYM> gives. A mirrored codebook
// searches |z| over the positive half and takes the mirrored cell for z < 0:
// the top bit is [z >= 0] and the others are the magnitude's bits, inverted for
// z < 0; every mask it returns is made by a scalar instruction. The general
// search returns the compare masks themselves.
template <int BITS, int SYM>
__device__ inline void code_masks(float z, const float* t, uint64_t (&m)[BITS]) {
  if constexpr (SYM) {
    const float* p = t + (1 << (BITS - 1));
    const uint64_t neg = lanes(z < 0.f);
    const float x = fabsf(z);
    m[BITS - 1] = ~neg;
    if constexpr (BITS == 2) {
      m[0] = lanes(x >= p[0]) ^ neg;
    } else if constexpr (BITS == 3) {
      const bool c1 = x >= p[1];
      const bool c0 = x >= (c1 ? p[2] : p[0]);
      m[1] = lanes(c1) ^ neg;
      m[0] = lanes(c0) ^ neg;
    } else {
      const bool c2 = x >= p[3];
      const bool c1 = x >= (c2 ? p[5] : p[1]);
      const float lo = c2 ? p[4] : p[0], hi = c2 ? p[6] : p[2];   // (flat selects, no branches)
      const bool c0 = x >= (c1 ? hi : lo);
      m[2] = lanes(c2) ^ neg;
      m[1] = lanes(c1) ^ neg;
      m[0] = lanes(c0) ^ neg;
    }
  } else {
    if constexpr (BITS == 2) {
      const bool c1 = z >= t[1];
      const bool c0 = z >= (c1 ? t[2] : t[0]);
      m[1] = lanes(c1);
      m[0] = lanes(c0);
    } else if constexpr (BITS == 3) {
      const bool c2 = z >= t[3];
      const bool c1 = z >= (c2 ? t[5] : t[1]);
      const float lo = c2 ? t[4] : t[0], hi = c2 ? t[6] : t[2];
      const bool c0 = z >= (c1 ? hi : lo);
      m[2] = lanes(c2);
      m[1] = lanes(c1);
      m[0] = lanes(c0);
    } else {
      const bool c3 = z >= t[7];
      const bool c2 = z >= (c3 ? t[11] : t[3]);
      const float a1 = c3 ? t[9] : t[1], b1 = c3 ? t[13] : t[5];
      const bool c1 = z >= (c2 ? b1 : a1);
      const float a0 = c3 ? t[8] : t[0], b0 = c3 ? t[10] : t[2], e0 = c3 ? t[12] : t[4], f0 = c3 ? t[14] : t[6];
      const float g0 = c2 ? e0 : a0, h0 = c2 ? f0 : b0;
      const bool c0 = z >= (c1 ? h0 : g0);
      m[3] = lanes(c3);
      m[2] = lanes(c2);
      m[1] = lanes(c1);
      m[0] = lanes(c0);
    }
  }
}

// Lanes i and i + 32 combine x (both get the result). The exchange runs
// through ds_bpermute: v_permlane32_swap on a just-copied register gave lanes
// 32-63 a stale copy here, with the wait states the compiler puts in front.
__device__ inline float sum_halves(float x) { return x + shfl_xor_f(x, 32); }
__device__ inline float max_halves(float x) { return fmaxf(x, shfl_xor_f(x, 32)); }

// Sum of squares of the 64 bfloat16 coordinates of a lane, two per
// v_dot2c_f32_bf16. (Written as an instruction: with this compiler the dot2
// builtin on bit-cast words reads the first word of each vector only.)
__device__ inline float sumsq_bf16(const RawX32<0>& r) {
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
#pragma unroll
    for (int w = 0; w < 4; ++w) asm("v_dot2c_f32_bf16 %0, %1, %1" : "+v"(ss) : "v"(r.v[k][w]));
  }
  return ss;
}

// One 32-coordinate output block jb of y = Pi x from NPART bfloat16 parts of Pi
// (3: the smallest first; 1: the signs of a one-magnitude matrix), the
// operands of step ks + 1 read from LDS while step ks runs.
template <int ROLE, int NPART>
__device__ inline floatx16 rotate_bf16(const u32x4* piop, const RawX32<0>& x, int jb, int lane) {
  floatx16 acc = {};
  const u32x4* blk = piop + qb_piece(jb, 0, 0) + lane;
  u32x4 cur[NPART], nxt[NPART];
  auto read = [&](int ks, u32x4(&o)[NPART]) {
#pragma unroll
    for (int q = 0; q < NPART; ++q) o[q] = blk[qb_piece(0, ks, NPART - 1 - q)];
  };
  read(0, cur);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (ks < 7) read(ks + 1, nxt);
#pragma unroll
    for (int q = 0; q < NPART; ++q) {
      if constexpr (ROLE == TQ_KEYS) acc = mfma32bf(cur[q], x.v[ks], acc);
      else acc = mfma32bf(x.v[ks], cur[q], acc);
    }
    if (ks < 7) {
#pragma unroll
      for (int q = 0; q < NPART; ++q) cur[q] = nxt[q];
    }
  }
  return acc;
}

// Where a wavefront's tile lies: its first slot is slot r0 of (row * H_kv +
// head) bh0. The walk advances by the grid stride with scalar adds, so no tile
// pays a 64-bit division (B and H_kv are below 2^16, so bh fits 32 bits).
struct SlotWalk {
  uint32_t bh0, r0;   // first slot of the current tile
  uint32_t dq, dr;    // the grid stride, in (heads, slots)
  __device__ void init(const QuantArgs& a, int64_t s0, int64_t stride) {
    bh0 = (uint32_t)(s0 / a.nslot);
    r0 = (uint32_t)(s0 - (int64_t)bh0 * a.nslot);
    dq = (uint32_t)(stride / a.nslot);
    dr = (uint32_t)(stride - (int64_t)dq * a.nslot);
  }
  __device__ void advance(const QuantArgs& a) {
    const uint32_t ns = (uint32_t)a.nslot;
    r0 += dr;
    bh0 += dq;
    if (r0 >= ns) {
      r0 -= ns;
      ++bh0;
    }
  }
  // (head, slot within the head) of slot v (< 32) of the tile; the slot's token
  // is t_base + r
  __device__ void at(const QuantArgs& a, uint32_t v, uint32_t& bh, uint32_t& r) const {
    const uint32_t ns = (uint32_t)a.nslot;
    const uint32_t rr = r0 + v;
    const uint32_t q = ns >= 32u ? (rr >= ns ? 1u : 0u) : rr / ns;
    bh = bh0 + q;
    r = rr - q * ns;
  }
};

// Whether slot (bh, r) holds an input vector.
__device__ inline bool slot_valid(const QuantArgs& a, uint32_t bh, uint32_t r) {
  const int64_t t = a.t_base + r;
  return (int64_t)bh < a.B * a.H_kv && t >= a.t_offset && t < a.t_offset + a.T;
}

// The lane's 64 coordinates 16ks + 8kh + e of the vector in slot (bh, sr).
__device__ inline void load_bf16(RawX32<0>& r, const QuantArgs& a, uint32_t bh, uint32_t sr, int kh) {
  const bool valid = slot_valid(a, bh, sr);
  r.valid = valid;
  if (valid) {
    const uint32_t hk = (uint32_t)a.H_kv;
    const uint32_t b = bh / hk, h = bh - b * hk;
    const int64_t off = (int64_t)b * a.sb + (a.t_base + sr - a.t_offset) * a.st + (int64_t)h * a.sh + 8 * kh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) r.v[ks] = *(const u32x4*)((const uint16_t*)a.x + off + 16 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) r.v[ks] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int BITS, int ROLE>
__global__ __launch_bounds__(64 * kQbWaves) void quantize_bf16_kernel(QuantArgs a) {
  constexpr int TILE = 32 * kQbWaves;
  constexpr int NT = (1 << BITS) - 1;
  extern __shared__ __align__(16) unsigned char smem[];
  u32x4* piop = (u32x4*)smem;                                 // [jb][ks][part][lane]
  float* fzs = (float*)(smem + 3 * kQbPart * sizeof(u32x4));   // [wave][32]: sqrt(d) / |x| by slot
  // (keys: then [wave][BITS][64] words of the first pass)

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i32 = lane & 31, kh = lane >> 5;
  const int slot = qb_slot<ROLE>(i32);
  const float csign = stage_matrix_bf16<ROLE>(a.rot, piop);
  __syncthreads();

  const Thresholds<BITS> th = load_thresholds<BITS>(a);
  const float sqrt_d = sqrtf((float)kD);

  // NPART = 3: the MFMAs give y itself; NPART = 1 (a one-magnitude rotation):
  // they give S x, and y = csign * (S x)
  auto tiles = [&](auto npart) __attribute__((always_inline)) {
  constexpr int NPART = decltype(npart)::value;
  const float yd = (NPART == 1 ? csign : 1.f) * sqrt_d;   // z = (MFMA output) * yd / |x|
  const float inv_yd = 1.f / yd;
  uint64_t sink = 0;   // carry-outs of the bit pushes (never read)
  SlotWalk walk;
  uint32_t bh = 0, sr = 0;   // the lane's vector: row * H_kv + head, slot within the head
  RawX32<0> cur;
  if (blockIdx.x < a.n_tiles) {
    walk.init(a, (int64_t)blockIdx.x * TILE + wave * 32, (int64_t)gridDim.x * TILE);
    walk.at(a, slot, bh, sr);
    load_bf16(cur, a, bh, sr, kh);
  }

  for (int64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
    RawX32<0> nxt;
    SlotWalk wnext = walk;
    uint32_t bh_n = 0, sr_n = 0;
    if (tile + gridDim.x < a.n_tiles) {
      wnext.advance(a);
      wnext.at(a, slot, bh_n, sr_n);
      load_bf16(nxt, a, bh_n, sr_n, kh);
    }

    // ---- norm (and a power-of-two rescale of vectors far from 1)
    float ss = sum_halves(sumsq_bf16(cur));
    int sexp = 0;
    const bool rescale = cur.valid && !(ss >= 0x1p-100f && ss <= 0x1p100f);
    if (lanes(rescale) != 0) {
      // (rare: one word at a time, so this path adds no register pressure)
      uint32_t mb = 0u;   // largest magnitude, as bfloat16 bits (ordered like the values)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t m = cur.v[k][w] & 0x7FFF7FFFu;
          mb = max(mb, max(m & 0xFFFFu, m >> 16));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const float mx = max_halves(__uint_as_float(mb << 16));
      sexp = (rescale && mx > 0.f) ? -__builtin_amdgcn_frexp_expf(mx) : 0;   // largest entry in [1/2, 1)
      if (sexp != 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = ldexpf(__uint_as_float(cur.v[k][w] << 16), sexp);
            const float hi = ldexpf(__uint_as_float(cur.v[k][w] & 0xFFFF0000u), sexp);
            cur.v[k][w] = bf16_bits(lo) | bf16_bits(hi) << 16;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      ss = sum_halves(sumsq_bf16(cur));
    }
    // |x| * 2^sexp, and sqrt(d) / that (single instructions, within 2 ulp: the
    // code decisions are tested outside a 1e-6 band around each threshold)
    const float ns = __builtin_amdgcn_sqrtf(ss);
    const float fz = ns > 0.f ? yd * __builtin_amdgcn_rcpf(ns) : 0.f;
    const int64_t row = cur.valid ? tok_row(a.pm, a.H_kv, a.T_cap, bh, a.t_base + sr) : -1;
    if (row >= 0 && kh == 0) a.norms[row] = ldexpf(ns, -sexp);

    if constexpr (ROLE == TQ_KEYS) {
      // Mirrored codebook: y against thresholds in units of y (the positive
      // half only, few registers). A zero vector (y = 0) belongs in the cell of
      // z = 0, #{t_i <= 0}: the floor on the scale keeps each threshold's sign
      // (nonzero norms are at least 2^-50 here, far above it). Any other
      // codebook: z = y sqrt(d) / |x| against the thresholds themselves.
      float ts[NT];
      const float sc = fmaxf(ns * inv_yd, 0x1p-100f);
#pragma unroll
      for (int i = 0; i < NT; ++i) ts[i] = th.t[i] * sc;
      auto run = [&](auto sym) {
        constexpr int SYM = decltype(sym)::value;
        // two output blocks (32 coordinates, BITS words) per pass; the lane's
        // 2 BITS words (its half of the token's row) leave in one store, so the
        // row's cache lines are written whole
        // pass 0's words wait in LDS ([BITS][64] per wavefront)
        uint32_t* w0 = (uint32_t*)(fzs + kQbWaves * 32) + wave * (64 * BITS) + lane;
#pragma unroll 1
        for (int p = 0; p < 2; ++p) {
          uint32_t w[BITS];
#pragma unroll
          for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
          for (int jj = 1; jj >= 0; --jj) {
            const int jb = 2 * p + jj;
            const floatx16 acc = rotate_bf16<ROLE, NPART>(piop, cur, jb, lane);
#pragma unroll
            for (int e = 15; e >= 0; --e) {
              uint64_t m[BITS];
              if constexpr (SYM) code_masks<BITS, 1>(acc[e], ts, m);
              else code_masks<BITS, 0>(acc[e] * fz, th.t, m);
#pragma unroll
              for (int k = BITS - 1; k >= 0; --k) {
                const int pos = BITS * (16 * jj + e) + k;
                w[pos >> 5] = push_bit<!SYM>(w[pos >> 5], m[k], sink);
              }
              if (e % 2 == 0) __builtin_amdgcn_sched_barrier(0);   // two codes' masks in flight at most
            }
          }
          if (p == 0) {
#pragma unroll
            for (int k = 0; k < BITS; ++k) w0[64 * k] = w[k];
          } else if (row >= 0) {
            uint32_t* dst = a.codes + row * (4 * BITS) + 2 * BITS * kh;
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[k] = w0[64 * k];
#pragma unroll
            for (int k = 0; k < BITS; ++k) dst[BITS + k] = w[k];
          }
        }
      };
      if (th.sym)
        run(IntTag<1>{});
      else
        run(IntTag<0>{});
    } else {
      if (kh == 0) fzs[wave * 32 + slot] = fz;
      wave_sync();
      // the lane's two 8-token blocks 2kh + bi: first row, and the bits of the
      // block's words that belong to tokens outside [t_offset, t_offset + T)
      const int qm = lane & 3;                       // word of the coordinate group this lane forms
      const int qa = (4 * qm) / BITS;                // first quad lane whose piece it needs
      const uint32_t sa = 32 * qm - 8 * BITS * qa;   // that piece's shift
      const uint32_t sb = 8 * BITS - sa;             // and the next one's
      int64_t brow[2];
      uint32_t keep[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        uint32_t bhb, srb;
        walk.at(a, 8 * (2 * kh + bi), bhb, srb);
        const int64_t tb = a.t_base + srb;
        int lo = 8, hi = 0;   // valid tokens [lo, hi) of the block
        if ((int64_t)bhb < a.B * a.H_kv) {
          const int64_t l = a.t_offset - tb, h = a.t_offset + a.T - tb;
          lo = (int)(l < 0 ? 0 : (l > 8 ? 8 : l));
          hi = (int)(h < 0 ? 0 : (h > 8 ? 8 : h));
        }
        brow[bi] = lo < hi ? tok_row(a.pm, a.H_kv, a.T_cap, bhb, tb) : -1;
        // per piece: bits of tokens below lo or from hi on
        const uint64_t piece_keep =
            ((1ull << (BITS * lo)) - 1ull) | (((1ull << (8 * BITS)) - 1ull) & ~((1ull << (BITS * (lo < hi ? hi : lo))) - 1ull));
        keep[bi] = BITS == 4 ? (uint32_t)piece_keep
                             : (uint32_t)(piece_keep >> sa) | (uint32_t)(piece_keep << sb);
      }
      auto run = [&](auto sym) {
        constexpr int SYM = decltype(sym)::value;
#pragma unroll 1
        for (int jb = 0; jb < 4; ++jb) {
          const floatx16 acc = rotate_bf16<ROLE, NPART>(piop, cur, jb, lane);
          uint32_t piece[2];
#pragma unroll
          for (int bi = 0; bi < 2; ++bi) {
            // sqrt(d) / |x| of the block's 8 vectors (an LDS broadcast, read per block)
            const float4* fz4 = (const float4*)(fzs + wave * 32 + 16 * kh + 8 * bi);
            const float4 f0 = fz4[0], f1 = fz4[1];
            const float fz[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
            uint32_t c = 0u;
#pragma unroll
            for (int ti = 7; ti >= 0; --ti) {
              uint64_t m[BITS];
              code_masks<BITS, SYM>(acc[8 * bi + ti] * fz[ti], th.t, m);
#pragma unroll
              for (int k = BITS - 1; k >= 0; --k) c = push_bit<!SYM>(c, m[k], sink);
              // (two codes' lane masks in flight at most: they live in scalar registers)
              if (ti % 2 == 0) __builtin_amdgcn_sched_barrier(0);
            }
            piece[bi] = c;
          }
          // quad merge: word qm of coordinate group 8jb + j/4 = bits [32qm, 32qm + 32) of the
          // concatenated pieces of coordinates 4cg .. 4cg+3 (8*BITS bits each)
          constexpr int PA = BITS == 2 ? 0x08 : 0xE4;   // quad lane of the first piece
          constexpr int PB = BITS == 2 ? 0x0D : 0xF9;   // and of the second
#pragma unroll
          for (int bi = 0; bi < 2; ++bi) {
            uint32_t word;
            if constexpr (BITS == 4) {
              word = piece[bi];
            } else {
              const uint32_t pa = BITS == 3 ? piece[bi] : (uint32_t)__builtin_amdgcn_mov_dpp((int)piece[bi], PA, 0xF, 0xF, false);
              const uint32_t pb = (uint32_t)__builtin_amdgcn_mov_dpp((int)piece[bi], PB, 0xF, 0xF, false);
              word = (pa >> sa) | (pb << sb);
            }
            if (qm < BITS && brow[bi] >= 0) {
              uint32_t* dst = a.codes + brow[bi] * (4 * BITS) + (8 * jb + (i32 >> 2)) * BITS + qm;
              *dst = keep[bi] == 0u ? word : ((*dst & keep[bi]) | (word & ~keep[bi]));
            }
          }
        }
      };
      if (th.sym)
        run(IntTag<1>{});
      else
        run(IntTag<0>{});
    }
    wave_sync();   // the scale buffer is rewritten by the next tile
    cur = nxt;
    walk = wnext;
    bh = bh_n;
    sr = sr_n;
  }
  asm volatile("" ::"s"(sink));   // the carry-out pair stays reserved to the end
  };
  if (csign > 0.f)
    tiles(IntTag<1>{});
  else
    tiles(IntTag<3>{});
}

// ------------------------------------------------- single-token append --
//
// One token per (row, head) (T = 1) without QJL: latency, not throughput,
// decides here, so the rotation runs as float32 FMAs with the rows of Pi read
// straight from memory in segments (rotate_rows, the arithmetic the decode
// kernel repeats when it appends the token itself; no LDS staging of Pi, no
// operand split), kAppendVecs
// vectors per 256-thread workgroup (few, so that a layer's tokens spread over
// many compute units and each thread's dot products stay short). Same steps as
// the tiled kernels: power-of-two scale, norm, y = Pi x, threshold search,
// packing (a value block keeps the bits of its other tokens).
constexpr int kAppendVecs = 1;

// The append of workgroup blk (vector blk = row * H_kv + head) of one cache,
// at token t (t < 0: nothing).
template <int BITS, int ROLE, int XF32>
__device__ void append_vectors(const QuantArgs& a, int64_t blk, int64_t t) {
  if (t < 0) return;   // (workgroup-uniform)
  static_assert(kAppendVecs == 1, "one vector per workgroup");
  __shared__ __align__(16) float xs[kD];
  __shared__ __align__(16) float ys[kD];
  __shared__ __align__(16) unsigned char cb[kD];
  __shared__ float fz[2];
  const int lt = threadIdx.x;
  AppendOne<BITS, ROLE> ap;
  RowSegment<256> rs;
  float x[4];
  load_row_segment<256>(rs, a.rot);
  ap.load_old(a, blk, t, lt);
  AppendOne<BITS, ROLE>::load_x(a, blk, lt, XF32 != 0, x);
  ap.begin(a, blk, t, lt, x, xs, fz);
  __syncthreads();
  rotate_rows<256, 1>(rs, xs, ys, 1);
  __syncthreads();
  if (lt < kD) AppendOne<BITS, ROLE>::encode_coord(load_thresholds<BITS>(a), lt, ys, fz, cb);
  __syncthreads();
  ap.finish(a, blk, t, lt, fz, cb);
}

template <int BITS, int ROLE, int XF32>
__global__ __launch_bounds__(256) void append_kernel(QuantArgs a) {
  append_vectors<BITS, ROLE, XF32>(a, blockIdx.x, a.t_offset);
}

// Keys and values of the same new token in one launch: the first nk
// workgroups append to the key cache, the rest to the value cache. With
// context lengths, row b's token goes to clamp(ctx_lens[b], 0, T) - 1 (none
// for an empty row), else to t_offset.
template <int KB, int VB, int XF32>
__global__ __launch_bounds__(256) void append_pair_kernel(QuantArgs ka, QuantArgs va, int64_t nk,
                                                          const int32_t* ctx_lens, int64_t T) {
  const bool key = (int64_t)blockIdx.x < nk;
  const int64_t blk = key ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - nk;
  int64_t t = ka.t_offset;
  if (ctx_lens != nullptr) {
    const int64_t c = ctx_lens[blk / ka.H_kv];
    t = (c < 0 ? 0 : (c > T ? T : c)) - 1;
  }
  if (key) append_vectors<KB, TQ_KEYS, XF32>(ka, blk, t);
  else append_vectors<VB, TQ_VALUES, XF32>(va, blk, t);
}

// ------------------------------------------------------------- dequantize --

struct DequantArgs {
  const uint32_t* codes;
  const float* norms;
  const uint32_t* signs;
  const float* gamma;
  const float* rot;
  const float* proj;
  float* out;
  int64_t H_kv, T_cap, t0, t1;
  float cent[16];
  PageMap pm;
};

template <int BITS, int ROLE, int QJL>
__global__ __launch_bounds__(256) void dequantize_kernel(DequantArgs a) {
  __shared__ float wv[32 * kD];
  __shared__ float sg[QJL ? 32 * kD : 1];
  __shared__ float nrm[32], gm[32];
  __shared__ int64_t rows[32];   // token rows of the block's tokens (-1: none)
  constexpr int KW = 4 * BITS;
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H_kv + h;
  const int64_t tbase = a.t0 + (int64_t)blockIdx.x * 32;
  const float inv_sqrt_d = 1.0f / sqrtf((float)kD);
  const uint32_t* cb = a.codes;
  if (tid < 32) {
    const int64_t t = tbase + tid;
    rows[tid] = t < a.t1 ? tok_row(a.pm, a.H_kv, a.T_cap, bh, t) : -1;
  }
  __syncthreads();
  for (int idx = tid; idx < 32 * kD; idx += 256) {
    const int v = idx / kD, j = idx % kD;
    const int64_t t = tbase + v;
    const int64_t row = rows[v];
    float val = 0.f;
    if (row >= 0) {
      int64_t bit;
      if constexpr (ROLE == TQ_KEYS) bit = row * KW * 32 + (int64_t)BITS * j;
      else bit = (row / 8) * (int64_t)(32 * BITS) * 32 + (int64_t)BITS * (8 * j + (row % 8));
      const int64_t wi = bit >> 5;
      const int off = (int)(bit & 31);
      uint32_t x = cb[wi] >> off;
      if (off + BITS > 32) x |= cb[wi + 1] << (32 - off);
      const int code = (int)(x & ((1u << BITS) - 1u));
      float cc = a.cent[0];
#pragma unroll
      for (int q = 1; q < (1 << BITS); ++q) cc = (code == q) ? a.cent[q] : cc;
      val = cc * inv_sqrt_d;
      if constexpr (QJL) {
        const uint32_t sw = a.signs[row * 4 + (j >> 5)];
        sg[idx] = ((sw >> (j & 31)) & 1u) ? 1.f : -1.f;
      }
    } else if constexpr (QJL) {
      sg[idx] = 0.f;
    }
    wv[idx] = val;
  }
  if (tid < 32) {
    const int64_t t = tbase + tid;
    const int64_t row = rows[tid];
    nrm[tid] = row >= 0 ? a.norms[row] : 0.f;
    if constexpr (QJL) gm[tid] = row >= 0 ? a.gamma[row] : 0.f;
  }
  __syncthreads();
  const int col = tid & 127, half = tid >> 7;   // output coordinate, vector half
  float acc[16];
  if constexpr (QJL) {
    // w += gamma sqrt(pi/2)/d * S^T sigma
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    for (int i = 0; i < kD; ++i) {
      const float s = a.proj[i * kD + col];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = fmaf(s, sg[(16 * half + v) * kD + i], acc[v]);
    }
    __syncthreads();
    const float cq = sqrtf((float)M_PI / 2.0f) / (float)kD;
#pragma unroll
    for (int v = 0; v < 16; ++v) wv[(16 * half + v) * kD + col] += gm[16 * half + v] * cq * acc[v];
    __syncthreads();
  }
  // x_hat = n Pi^T w
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  for (int j = 0; j < kD; ++j) {
    const float p = a.rot[j * kD + col];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = fmaf(p, wv[(16 * half + v) * kD + j], acc[v]);
  }
  const int64_t nt = a.t1 - a.t0;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t t = tbase + 16 * half + v;
    if (t < a.t1) a.out[(bh * nt + (t - a.t0)) * kD + col] = nrm[16 * half + v] * acc[v];
  }
}

// Compute units of the current device (a per-device cache of a constant
// attribute; concurrent first calls store the same value).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int BITS, int ROLE, int QJL, int XF32>
hipError_t launch_q(const QuantArgs& qa, hipStream_t stream) {
  constexpr int WAVES = quant_waves<QJL>();
  constexpr size_t OPH = 4 * 8 * 64 * 8;
  constexpr size_t smem = (QJL ? 4 : 2) * OPH * 2 + WAVES * 16 * kD + (QJL ? WAVES * 2 * 16 * kD * 2 : 0);
  auto kern = quantize_kernel<BITS, ROLE, QJL, XF32>;
  // more than 64 KB of dynamic LDS needs the opt-in, once per process
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  const int per_cu = QJL ? 1 : 2;   // workgroups that fit a compute unit's 160 KB of LDS
  int64_t grid = (int64_t)compute_units() * per_cu;
  if (grid > qa.n_tiles) grid = qa.n_tiles;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * WAVES), smem, stream, qa);
  return hipGetLastError();
}

template <int BITS, int ROLE, int XF32>
hipError_t launch_q32(const QuantArgs& qa, hipStream_t stream) {
  constexpr size_t smem = 2 * kQ32OpHalves * 2 + kQ32Waves * 32 * kQ32Row;
  auto kern = quantize32_kernel<BITS, ROLE, XF32>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  int64_t grid = compute_units();   // one workgroup (16 wavefronts, ~130 KB of LDS) per compute unit
  if (grid > qa.n_tiles) grid = qa.n_tiles;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kQ32Waves), smem, stream, qa);
  return hipGetLastError();
}

template <int BITS, int ROLE>
hipError_t launch_qbf(const QuantArgs& qa, hipStream_t stream) {
  static_assert(kQbWaves == kQ32Waves, "the tile loader assumes 32 * kQ32Waves slots per tile");
  constexpr size_t smem = 3 * kQbPart * sizeof(u32x4) + kQbWaves * 32 * sizeof(float) +
                          (ROLE == TQ_KEYS ? kQbWaves * 64 * BITS * sizeof(uint32_t) : 0);
  auto kern = quantize_bf16_kernel<BITS, ROLE>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (attr != hipSuccess) return attr;
  int64_t grid = compute_units();   // one workgroup (16 wavefronts, ~98 KB of LDS) per compute unit
  if (grid > qa.n_tiles) grid = qa.n_tiles;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kQbWaves), smem, stream, qa);
  return hipGetLastError();
}

// Bulk work (at least one 512-slot tile per compute unit) takes the 32-vector
// tiles (bfloat16 input on bfloat16 MFMAs, float32 input split into float16
// hi + lo); short appends take the 16-vector tiles, which spread the same
// slots over 4x more workgroups and finish sooner.
template <int BITS, int ROLE, int QJL>
hipError_t dispatch_x(int xf32, QuantArgs qa, hipStream_t s) {
  if constexpr (!QJL) {
    const int64_t slots = qa.B * qa.H_kv * qa.nslot;
    const int64_t tiles32 = (slots + 32 * kQ32Waves - 1) / (32 * kQ32Waves);
    if (tiles32 >= compute_units()) {
      qa.n_tiles = tiles32;
      return xf32 ? launch_q32<BITS, ROLE, 1>(qa, s) : launch_qbf<BITS, ROLE>(qa, s);
    }
  }
  const int64_t tile16 = 16 * quant_waves<QJL>();
  qa.n_tiles = (qa.B * qa.H_kv * qa.nslot + tile16 - 1) / tile16;
  return xf32 ? launch_q<BITS, ROLE, QJL, 1>(qa, s) : launch_q<BITS, ROLE, QJL, 0>(qa, s);
}

template <int BITS>
hipError_t dispatch_role(int role, int qjl, int xf32, const QuantArgs& qa, hipStream_t s) {
  if (role == TQ_VALUES) return dispatch_x<BITS, TQ_VALUES, 0>(xf32, qa, s);
  return qjl ? dispatch_x<BITS, TQ_KEYS, 1>(xf32, qa, s) : dispatch_x<BITS, TQ_KEYS, 0>(xf32, qa, s);
}

template <int BITS, int ROLE, int QJL>
hipError_t launch_dq(const DequantArgs& da, int64_t B, hipStream_t stream) {
  const int64_t n = da.t1 - da.t0;
  dim3 grid((unsigned)((n + 31) / 32), (unsigned)da.H_kv, (unsigned)B);
  hipLaunchKernelGGL((dequantize_kernel<BITS, ROLE, QJL>), grid, dim3(256), 0, stream, da);
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_dq(int role, int qjl, const DequantArgs& da, int64_t B, hipStream_t s) {
  if (role == TQ_VALUES) return launch_dq<BITS, TQ_VALUES, 0>(da, B, s);
  return qjl ? launch_dq<BITS, TQ_KEYS, 1>(da, B, s) : launch_dq<BITS, TQ_KEYS, 0>(da, B, s);
}

template <int BITS, int ROLE, int XF32>
hipError_t launch_append(const QuantArgs& qa, hipStream_t stream) {
  const int64_t grid = (qa.B * qa.H_kv + kAppendVecs - 1) / kAppendVecs;
  hipLaunchKernelGGL((append_kernel<BITS, ROLE, XF32>), dim3((unsigned)grid), dim3(256), 0, stream, qa);
  return hipGetLastError();
}

template <int BITS>
hipError_t dispatch_append(int role, int xf32, const QuantArgs& qa, hipStream_t s) {
  if (role == TQ_VALUES) return xf32 ? launch_append<BITS, TQ_VALUES, 1>(qa, s) : launch_append<BITS, TQ_VALUES, 0>(qa, s);
  return xf32 ? launch_append<BITS, TQ_KEYS, 1>(qa, s) : launch_append<BITS, TQ_KEYS, 0>(qa, s);
}

}  // namespace

QuantArgs make_quant_args(const void* x, int64_t B, int64_t T, int64_t H_kv, int64_t sb, int64_t st, int64_t sh,
                          const tq_cache* dst, int64_t t_offset) {
  QuantArgs qa;
  qa.x = x;
  qa.sb = sb;
  qa.st = st;
  qa.sh = sh;
  qa.B = B;
  qa.T = T;
  qa.H_kv = H_kv;
  qa.T_cap = dst->T_cap;
  qa.t_offset = t_offset;
  qa.t_base = (t_offset / kValueBlock) * kValueBlock;
  const int64_t t_hi = ((t_offset + T + kValueBlock - 1) / kValueBlock) * kValueBlock;
  qa.nslot = t_hi - qa.t_base;
  qa.n_tiles = 0;   // set by the dispatch, which picks the tile shape
  qa.codes = dst->codes;
  qa.norms = dst->norms;
  qa.signs = dst->qjl_signs;
  qa.gamma = dst->qjl_gamma;
  qa.rot = dst->rot;
  qa.proj = dst->qjl_proj;
  qa.pm = page_map(dst);
  const int L = 1 << dst->bits;
  for (int i = 0; i < 16; ++i) qa.cent[i] = i < L ? dst->centroids[i] : 0.f;
  thresholds_from_centroids(dst->centroids, L, qa.thr);
  for (int i = L - 1; i < 16; ++i) qa.thr[i] = INFINITY;
  qa.thr_sym = qa.thr[L / 2 - 1] == 0.0f;
  for (int k = 0; k < L / 2 - 1; ++k) qa.thr_sym &= qa.thr[L - 2 - k] == -qa.thr[k];
  return qa;
}

namespace {

template <int KB, int VB>
hipError_t launch_append_pair(int xf32, const QuantArgs& ka, const QuantArgs& va, const int32_t* ctx_lens,
                              int64_t T, hipStream_t stream) {
  const int64_t nk = (ka.B * ka.H_kv + kAppendVecs - 1) / kAppendVecs;
  const int64_t nv = (va.B * va.H_kv + kAppendVecs - 1) / kAppendVecs;
  if (xf32)
    hipLaunchKernelGGL((append_pair_kernel<KB, VB, 1>), dim3((unsigned)(nk + nv)), dim3(256), 0, stream, ka, va, nk,
                       ctx_lens, T);
  else
    hipLaunchKernelGGL((append_pair_kernel<KB, VB, 0>), dim3((unsigned)(nk + nv)), dim3(256), 0, stream, ka, va, nk,
                       ctx_lens, T);
  return hipGetLastError();
}

template <int KB>
hipError_t dispatch_pair(int vbits, int xf32, const QuantArgs& ka, const QuantArgs& va, const int32_t* ctx_lens,
                         int64_t T, hipStream_t s) {
  switch (vbits) {
    case 2: return launch_append_pair<KB, 2>(xf32, ka, va, ctx_lens, T, s);
    case 3: return launch_append_pair<KB, 3>(xf32, ka, va, ctx_lens, T, s);
    default: return launch_append_pair<KB, 4>(xf32, ka, va, ctx_lens, T, s);
  }
}

}  // namespace

hipError_t launch_quantize(const void* x, int x_dtype, int64_t B, int64_t T, int64_t H_kv,
                           int64_t sb, int64_t st, int64_t sh, const tq_cache* dst, int64_t t_offset,
                           hipStream_t stream) {
  const QuantArgs qa = make_quant_args(x, B, T, H_kv, sb, st, sh, dst, t_offset);
  const int xf32 = x_dtype == TQ_F32;
  const int qjl = dst->role == TQ_KEYS && dst->qjl;
  if (T == 1 && !qjl) {
    switch (dst->bits) {
      case 2: return dispatch_append<2>(dst->role, xf32, qa, stream);
      case 3: return dispatch_append<3>(dst->role, xf32, qa, stream);
      default: return dispatch_append<4>(dst->role, xf32, qa, stream);
    }
  }
  switch (dst->bits) {
    case 2: return dispatch_role<2>(dst->role, qjl, xf32, qa, stream);
    case 3: return dispatch_role<3>(dst->role, qjl, xf32, qa, stream);
    default: return dispatch_role<4>(dst->role, qjl, xf32, qa, stream);
  }
}

hipError_t launch_append_kv(const void* k, const void* v, int x_dtype, int64_t B, int64_t H_kv, int64_t k_sb,
                            int64_t k_sh, int64_t v_sb, int64_t v_sh, const tq_cache* kc, const tq_cache* vc,
                            int64_t t_offset, hipStream_t stream, const int32_t* ctx_lens, int64_t T) {
  if (kc->qjl) {
    // (the caller passes no context lengths with QJL keys)
    // keys with a QJL sketch take the tiled kernel: two launches
    const hipError_t e = launch_quantize(k, x_dtype, B, 1, H_kv, k_sb, 0, k_sh, kc, t_offset, stream);
    if (e != hipSuccess) return e;
    return launch_quantize(v, x_dtype, B, 1, H_kv, v_sb, 0, v_sh, vc, t_offset, stream);
  }
  const QuantArgs ka = make_quant_args(k, B, 1, H_kv, k_sb, 0, k_sh, kc, t_offset);
  const QuantArgs va = make_quant_args(v, B, 1, H_kv, v_sb, 0, v_sh, vc, t_offset);
  const int xf32 = x_dtype == TQ_F32;
  switch (kc->bits) {
    case 2: return dispatch_pair<2>(vc->bits, xf32, ka, va, ctx_lens, T, stream);
    case 3: return dispatch_pair<3>(vc->bits, xf32, ka, va, ctx_lens, T, stream);
    default: return dispatch_pair<4>(vc->bits, xf32, ka, va, ctx_lens, T, stream);
  }
}

hipError_t launch_dequantize(const tq_cache* src, int64_t t0, int64_t t1, float* out, hipStream_t stream) {
  DequantArgs da;
  da.codes = src->codes;
  da.norms = src->norms;
  da.signs = src->qjl_signs;
  da.gamma = src->qjl_gamma;
  da.rot = src->rot;
  da.proj = src->qjl_proj;
  da.out = out;
  da.H_kv = src->H_kv;
  da.T_cap = src->T_cap;
  da.pm = page_map(src);
  da.t0 = t0;
  da.t1 = t1;
  const int L = 1 << src->bits;
  for (int i = 0; i < 16; ++i) da.cent[i] = i < L ? src->centroids[i] : 0.f;
  const int qjl = src->role == TQ_KEYS && src->qjl;
  switch (src->bits) {
    case 2: return dispatch_dq<2>(src->role, qjl, da, src->B, stream);
    case 3: return dispatch_dq<3>(src->role, qjl, da, src->B, stream);
    default: return dispatch_dq<4>(src->role, qjl, da, src->B, stream);
  }
}

}  // namespace tq
