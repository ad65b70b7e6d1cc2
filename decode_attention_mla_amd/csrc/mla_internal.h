// Internal declarations shared by the host planner and the HIP translation unit.
#pragma once

#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {

constexpr int kPage = 64;       // tokens per KV page
constexpr int kDqk = 576;       // 512 latent + 64 RoPE dims (QK^T)
constexpr int kDv = 512;        // latent dims (PV)
constexpr int kSmallRows = 16;  // up to this many query rows: one workgroup covers them all
constexpr int kRowGroup = 32;   // query rows per workgroup above that
constexpr int kWideRows = 128;  // from this many rows on: workgroups of 128 rows

// 64-token pages of a sequence of L >= 0 tokens, ceil(L / 64) without the
// int32 overflow of (L + 63) / 64 for L > 2^31 - 64; 0 for L <= 0.
constexpr int pages_of(int L) { return L > 0 ? (L >> 6) + ((L & (kPage - 1)) != 0) : 0; }

// Records `code` and a printf-style message as this thread's last error; returns `code`.
int set_error(int code, const char* fmt, ...);

int plan(const int32_t* seqlens, int batch, int num_parts, int fixed_overhead, int force_splits,
         int32_t* sched, int max_parts, int32_t* num_splits, int* parts_out);
int attach_pages(int32_t* sched, int num_parts, const int32_t* seqlens, int batch, const int32_t* block_table,
                 int max_blocks, int num_blocks);

// Launch geometry shared by the planner policy and the kernels.
struct Geometry {
  int R;           // query rows per request = s_q * h_q
  int row_groups;  // workgroups per part: 1 for R <= 16, ceil(R / 128) for R >= 128 (or an FP8 cache),
                   // else ceil(R / 32)
};

// An FP8 cache takes the 128-row kernel for every R above 16 (the 32-row
// kernel has no FP8 variant), so its plan uses that geometry.
inline Geometry geometry(int h_q, int s_q, bool fp8) {
  Geometry g;
  g.R = h_q * s_q;
  g.row_groups = g.R <= kSmallRows                 ? 1
                 : (g.R >= kWideRows || fp8)       ? (g.R + kWideRows - 1) / kWideRows
                                                   : (g.R + kRowGroup - 1) / kRowGroup;
  return g;
}

// Sparse decode: every (request, query token) has its own key list, so a
// "request" of the split-KV kernels is one (request, query token) with
// R = h_q rows; above 16 rows it takes the 128-row kernel.
inline Geometry geometry_sparse(int h_q) {
  Geometry g;
  g.R = h_q;
  g.row_groups = g.R <= kSmallRows ? 1 : (g.R + kWideRows - 1) / kWideRows;
  return g;
}

}  // namespace mla
