// Internal declarations shared by the host planner and the HIP translation unit.
#pragma once

#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {

constexpr int kPage = 64;     // tokens per KV page
constexpr int kDqk = 576;     // 512 latent + 64 RoPE dims (QK^T)
constexpr int kDv = 512;      // latent dims (PV)
constexpr int kRowTile = 32;  // query rows per wave (one 32x32 MFMA column block)
constexpr int kMaxWaves = 4;  // waves per workgroup, one per SIMD

// Records `code` and a printf-style message as this thread's last error; returns `code`.
int set_error(int code, const char* fmt, ...);

int plan(const int32_t* seqlens, int batch, int num_parts, int fixed_overhead, int force_splits,
         int32_t* sched, int max_parts, int32_t* num_splits, int* parts_out);

// Launch geometry shared by the planner policy and the kernels.
struct Geometry {
  int R;           // query rows per request = s_q * h_q
  int row_tiles;   // ceil(R / 32)
  int waves;       // waves per workgroup (each owns one 32-row tile)
  int row_groups;  // workgroups per part = ceil(row_tiles / waves)
};

inline Geometry geometry(int h_q, int s_q) {
  Geometry g;
  g.R = h_q * s_q;
  g.row_tiles = (g.R + kRowTile - 1) / kRowTile;
  // 1, 2 or 4 waves: each wave owns 16 / waves of the 512 output columns.
  g.waves = g.row_tiles >= 3 ? kMaxWaves : g.row_tiles;
  g.row_groups = (g.row_tiles + g.waves - 1) / g.waves;
  return g;
}

}  // namespace mla
