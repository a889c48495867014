// Internal declarations shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kD = 128;              // head dimension this build supports
constexpr int kValueBlock = 8;       // tokens per value-layout block
constexpr int kStep = 32;            // tokens per decode inner step
constexpr int kChunkQuantum = 512;   // context chunks are whole multiples of this many tokens
                                     // (whole steps for each of up to 16 wavefronts)
constexpr int kDecodeTargetWGs = 256;   // one workgroup per compute unit of a 256-CU part

// Decode planning shared by the workspace-size helper and the launcher.
struct DecodePlan {
  int64_t B, H_q, H_kv, T;
  int32_t G;           // query heads per KV head
  int32_t wide;        // 0: G <= 8 (hi/lo query halves share one 16-column MFMA tile), 1: 8 < G <= 16
  int32_t qjl;
  int32_t n_split;     // context chunks per (row, KV head)
  int32_t chunk;       // tokens per chunk, multiple of kStep
  size_t off_ml, off_acc, bytes;   // chunk partials (used when n_split > 1)
};

bool plan_decode(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int32_t n_split, int32_t qjl,
                 DecodePlan* p);

// Host-side codebook helpers (tq_host.cpp).
void thresholds_from_centroids(const float* c, int levels, float* t);

// Launchers (return hipError_t of the launch).
hipError_t launch_quantize(const void* x, int x_dtype, int64_t B, int64_t T, int64_t H_kv,
                           int64_t sb, int64_t st, int64_t sh, const tq_cache* dst, int64_t t_offset,
                           hipStream_t stream);
hipError_t launch_dequantize(const tq_cache* src, int64_t t0, int64_t t1, float* out, hipStream_t stream);
hipError_t launch_decode(const DecodePlan& p, const tq_cache* k, const tq_cache* v, const void* q,
                         int q_dtype, const int32_t* ctx_lens, float scale, float* out, void* ws,
                         hipStream_t stream);

}  // namespace tq
