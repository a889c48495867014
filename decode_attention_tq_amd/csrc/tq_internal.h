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
  int64_t M;           // query tokens per row (1: decode; M > 1: chunked causal attention)
  int32_t Mt, nqt;     // query tokens per workgroup tile, tiles per row
  int32_t G;           // query heads per KV head
  int32_t wide;        // 0: Mt*G <= 8 (hi/lo query halves share one 16-column MFMA tile), 1: up to 16 columns
  int32_t qjl;
  int32_t n_split;     // context chunks per (row, KV head)
  int32_t chunk;       // tokens per chunk, multiple of kStep
  size_t off_ml, off_acc, bytes;   // chunk partials (used when n_split > 1)
};

// M query tokens per row (1 = decode). Columns of a workgroup are (query token,
// head) pairs: M*G <= 8 runs the 16-wavefront tile with all M tokens; more
// columns take the 16-column tile (8 wavefronts) with floor(16/G) tokens per
// tile.
bool plan_decode(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int32_t n_split, int32_t qjl,
                 DecodePlan* p, int64_t M = 1, int32_t d = kD);

// Dense chunked-prefill planning: every wavefront takes kDenseWaveCols
// (token, head) columns of one KV head, a workgroup 1, 2 or 4 wavefronts
// (nwave) that scan the same context chunk; ncg column groups per (row, KV
// head); n_split context chunks, merged (and rotated back) by the decode's
// combine kernel.
constexpr int kDenseWaveCols = 32;
struct DensePlan {
  int64_t B, H_q, H_kv, T, M;
  int32_t G, NC, nwave, ncg, n_split, chunk;
  size_t off_ml, off_acc, bytes;   // chunk partials [B*M*H_q][n_split][2], [..][d]
};

// The dense kernel takes chunked attention without QJL keys once the columns
// (M tokens x G heads) exceed one 16-column tile of the decode kernel.
inline bool use_dense_prefill(int64_t M, int64_t G, int32_t qjl) { return qjl == 0 && M > 1 && M * G > 16; }

bool plan_prefill_dense(int64_t B, int64_t H_q, int64_t H_kv, int64_t T, int64_t M, int32_t n_split, DensePlan* p);

// Block table of a cache in the paged layout; table == nullptr for the
// contiguous layout. Token t of (row b, head h) is token row
// (table[b][t >> lg] * H_kv + h) * 2^lg + t % 2^lg of the arrays.
struct PageMap {
  const int32_t* table;   // [B][maxblk] physical block of each logical block
  int64_t maxblk;         // logical blocks per row: T_cap >> lg
  int64_t nblk;           // physical blocks in the arrays
  int32_t lg;             // log2(block_tokens)
};

inline PageMap page_map(const tq_cache* c) {
  PageMap m{nullptr, 0, 0, 0};
  if (c->block_table != nullptr) {
    m.table = c->block_table;
    m.nblk = c->n_blocks;
    while ((int64_t(1) << m.lg) < c->block_tokens) ++m.lg;
    m.maxblk = c->T_cap >> m.lg;
  }
  return m;
}

// Token rows in a cache's arrays (B*H_kv*T_cap contiguous, n_blocks*H_kv*block_tokens paged).
inline int64_t cache_rows(const tq_cache* c) {
  return c->block_table != nullptr ? c->n_blocks * c->H_kv * c->block_tokens : c->B * c->H_kv * c->T_cap;
}

// Host-side codebook helpers (tq_host.cpp).
void thresholds_from_centroids(const float* c, int levels, float* t);

// Launchers (return hipError_t of the launch).
hipError_t launch_quantize(const void* x, int x_dtype, int64_t B, int64_t T, int64_t H_kv,
                           int64_t sb, int64_t st, int64_t sh, const tq_cache* dst, int64_t t_offset,
                           hipStream_t stream);
// (ctx_lens != NULL: row b's token goes to clamp(ctx_lens[b], 0, T) - 1, none
// for an empty row; no QJL keys then)
hipError_t launch_append_kv(const void* k, const void* v, int x_dtype, int64_t B, int64_t H_kv, int64_t k_sb,
                            int64_t k_sh, int64_t v_sb, int64_t v_sh, const tq_cache* kc, const tq_cache* vc,
                            int64_t t_offset, hipStream_t stream, const int32_t* ctx_lens = nullptr,
                            int64_t T = 0);
hipError_t launch_dequantize(const tq_cache* src, int64_t t0, int64_t t1, float* out, hipStream_t stream);
// Head dimensions 64 and 256 (tq_generic.hip). Quantize: ctx_lens == nullptr
// writes tokens [t_offset, t_offset + T); otherwise row b's single token x[b][0]
// goes to clamp(ctx_lens[b], 0, T_all) - 1 (none when that is -1).
hipError_t launch_quantize_generic(const void* x, int x_dtype, int64_t B, int64_t T, int64_t H_kv, int64_t sb,
                                   int64_t st, int64_t sh, const tq_cache* dst, int64_t t_offset,
                                   const int32_t* ctx_lens, int64_t T_all, hipStream_t stream);
hipError_t launch_dequantize_generic(const tq_cache* src, int64_t t0, int64_t t1, float* out, hipStream_t stream);
hipError_t launch_decode_generic(const tq_cache* k, const tq_cache* v, const void* q, int q_dtype, int64_t H_q,
                                 const int32_t* ctx_lens, int64_t T, float scale, float* out, hipStream_t stream);
// New key and value vectors of a decode step: element (b, h, j) at
// k[b*k_sb + h*k_sh + j] (and the same for v).
struct DecodeAppend {
  const void* k;
  const void* v;
  int x_dtype;
  int64_t k_sb, k_sh, v_sb, v_sh;
};
// Streaming-read reference (measurement helper): reads bytes of src once,
// one XOR-folded word per workgroup into sink.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                              hipStream_t stream);
hipError_t launch_prefill_dense(const DensePlan& p, const tq_cache* k, const tq_cache* v, const void* q, int q_dtype,
                                const int32_t* ctx_lens, float scale, float* out, void* ws, hipStream_t stream);
// Fixed-order merge of context-chunk partials of nvec query vectors
// ([nvec][n_split][2]: m, l; [nvec][n_split][d]: sums in the output basis)
// into out [nvec][d].
hipError_t launch_merge(const float* ml, const float* acc, float* out, int64_t nvec, int n_split, int d,
                        hipStream_t stream);
// app: the new token's key and value, quantized and appended by the decode
// kernel itself (d = 128 keys without a QJL sketch; the caller checks)
hipError_t launch_decode(const DecodePlan& p, const tq_cache* k, const tq_cache* v, const void* q,
                         int q_dtype, const int32_t* ctx_lens, float scale, float* out, void* ws,
                         hipStream_t stream, const DecodeAppend* app = nullptr);

}  // namespace tq
