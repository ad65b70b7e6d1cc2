// Dense MLA decode for MI355X (gfx950): split-KV main kernel, log-sum-exp
// combine kernel and the C ABI around them.
//
// What is computed (the "[DeepSeek-3] FlashMLA" overview page, sections 3-7):
// each request's s_q*h_q query rows (576 dims, weight-absorbed) attend over the
// request's paged 576-dim cache rows; QK^T uses all 576 dims, PV the first 512.
// A part of the launch grid walks a range of (request, 64-token block) work
// from the host planner; every piece is reduced with online softmax and either
// written out directly or, when its request is split across parts, stored as
// a normalised partial (O_i, lse_i) that the combine kernel merges.
//
// Kernel design (gfx950, not a translation of the pages' Hopper kernel):
//   * One workgroup per (part, group of up to 128 query rows), one wave per
//     SIMD; wave w owns a 32-row tile of queries.
//   * KV pages are copied HBM -> LDS with global_load_lds_dwordx4 (16 B per
//     lane straight into LDS), double buffered (2 x 72 KiB).  In LDS a page is
//     stored as 9 blocks of 64 dims; block b holds a 128-byte row per token
//     (dims 64b..64b+63) whose eight 16-byte chunks are permuted by a function
//     of the token so that both LDS read patterns below hit distinct banks.
//   * QK^T is computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K fragments come from LDS (ds_read_b128), Q fragments stay in registers
//     for the whole piece.  In the accumulator layout every lane then holds
//     one query row, so row max / row sum need one cross-half exchange and
//     the probabilities are already laid out as the B operand of the PV MFMA.
//   * PV is computed as O^T = V^T P^T; V^T fragments are read with
//     ds_read_b64_tr_b16 (transposing LDS read) from the same LDS page.
//   * Softmax runs in base 2 with log2(e) folded into the score scale (the
//     exp2 detail of the FlashMLA new-kernel deep-dive page).  Instead of
//     moving the running max every page and rescaling O (which would drag the
//     256-register accumulator through VALU each page), each piece keeps the
//     first page's row max as its reference: probabilities are 2^(s - m_ref)
//     and may exceed 1.  This is the online-softmax algebra with a fixed
//     reference, exact up to rounding.  If a row's max ever rises more than
//     64 (log2) above its reference, the workgroup restarts the piece with the
//     largest max seen so far as the new reference (a slow path that ordinary
//     inputs never take), so nothing can overflow.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "mla_internal.h"

namespace mla {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kChunks = kDqk / 8;                  // 72 sixteen-byte chunks per token row
constexpr int kRowBytes = kDqk * 2;                // 1152
constexpr int kPageBytes = kPage * kRowBytes;      // 73728
constexpr int kSlices = kPageBytes / 1024;         // 72 wave-wide 1 KiB copies per page
constexpr int kKSteps = kDqk / 16;                 // 36 MFMA k-steps for QK^T
constexpr int kColTiles = kDv / 32;                // 16 output column tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefHeadroom = 64.0f;              // log2 units a row max may exceed its reference
constexpr int kMaxRestarts = 16;                   // restarts per piece before giving up on headroom

struct Params {
  const unsigned char* q;      // bf16 [batch, R, 576]
  const unsigned char* kv;     // bf16 [num_blocks, 64, 576]
  const int32_t* block_table;  // [batch, max_blocks]
  const int32_t* seqlens;      // [batch]
  const int32_t* sched;        // [num_parts, 8]
  const int32_t* num_splits;   // [batch + 1] exclusive prefix
  unsigned short* out;         // bf16 [batch, R, 512]
  float* lse;                  // [batch, h_q, s_q]
  float* oacc;                 // [slots, row_tiles, 16, 64, 16] normalised partial O
  float* lacc;                 // [slots, row_tiles * 32] partial lse, base 2
  int R, h_q, s_q, max_blocks, num_parts, row_groups, row_tiles;
  float scale_log2;            // softmax_scale * log2(e)
};

// Chunk permutation of token row t inside an LDS column block: logical chunk
// c (0..7) of the row sits at position c ^ chunk_xor(t) (an involution).  It
// is a function of (t >> 1) & 7 chosen so that 16 consecutive tokens at one
// chunk, and the 4-token x 2-chunk footprint of a transposing read, each fall
// on distinct 16-byte bank groups (row stride 128 B = 8 groups of 16 B).
__device__ __forceinline__ int chunk_xor(int t) {
  const int x = (t >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

constexpr int kBlockBytes = kPage * 128;           // one 64-dim column block of a page (8 KiB)
constexpr int kPBufBytes = 4 * 4 * 64 * 16;        // bf16 P fragments: 4 row tiles x 4 k-steps x 64 lanes x 16 B

__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
  return (unsigned short)(u >> 16);
}

constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt not waited

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Asserts to the compiler that a pointer is the same in every lane (it is
// derived from wave-uniform values) so it can live in SGPRs.
__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const unsigned char*)(((unsigned long long)hi << 32) | lo);
}

// Per-lane global byte offset, inside a page, of the 16 bytes that lane l
// copies for an LDS slice of parity `par`: slice i (1 KiB = 64 x 16 B) of the
// LDS image is column block i / 8, tokens 8 (i % 8) + l / 8, chunk position
// l % 8; the token's permutation only depends on i % 2 and l / 16.
__device__ __forceinline__ unsigned dma_lane_offset(int lane, int par) {
  // Token 8 (i % 8) + lane / 8 has the same permutation as 8 par + lane / 8.
  const int cx = chunk_xor(8 * par + (lane >> 3));
  return (unsigned)((lane >> 3) * kRowBytes + (((lane & 7) ^ cx) << 4));
}

// Copy slice k of this wave's share of a 64x576 bf16 page to LDS: wave w
// owns slices w, w + NW, ... (72 / NW of them).  ``page`` must be uniform.
template <int NW>
__device__ __forceinline__ void issue_slice(const unsigned char* page, unsigned lds_base,
                                            const unsigned dma_off[2], int wave, int k) {
  const int i = wave + k * NW;
  // The opaque copy keeps the compiler from hoisting all 72/NW offsets out
  // of the page loop (they would stay live in VGPRs for the whole kernel).
  unsigned lane_off = dma_off[i & 1];
  asm volatile("" : "+v"(lane_off));
  const unsigned voff = lane_off + (unsigned)((i & 7) * 8 * kRowBytes + (i >> 3) * 128);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_base + (unsigned)i * 1024u);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(page),
               "s"(m0)
               : "memory");
}

// Copy one whole page (all of this wave's slices) to LDS.
template <int NW>
__device__ __forceinline__ void issue_page(const unsigned char* page_any, unsigned lds_base,
                                           const unsigned dma_off[2], int wave) {
  const unsigned char* page = uniform_ptr(page_any);
#pragma unroll
  for (int k = 0; k < kSlices / NW; ++k) issue_slice<NW>(page, lds_base, dma_off, wave, k);
}

// Wave-uniform read of read-only metadata through the constant address
// space, so it becomes a scalar load (lgkmcnt) and never waits on vmcnt,
// which counts the page copies in flight.
template <class T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)ptr;
}

__device__ __forceinline__ void map_block(const Params& p, int& part, int& rg) {
  const int id = blockIdx.x;
  if (p.row_groups == 1) {
    part = id;
    rg = 0;
    return;
  }
  // Keep the row groups of one part on the same XCD (workgroups are dealt to
  // the 8 XCDs round robin) and adjacent in dispatch order, so the second
  // reader of every KV page finds it in that XCD's L2.
  const int xcd = id & 7, slot = id >> 3;
  rg = slot % p.row_groups;
  part = (slot / p.row_groups) * 8 + xcd;
}

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1) mla_splitkv_kernel(Params p) {
  // Two KV page buffers plus the P exchange buffer: exactly 160 KiB.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[kPBufBytes];
  constexpr int kCtPerWave = kColTiles / NW;   // output column tiles owned by each wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, rg;
  map_block(p, part, rg);
  if (part >= p.num_parts) return;

  const int32_t* sp = p.sched + part * MLA_SCHED_INTS;
  const int begin_req = ld_uniform(sp), end_req = ld_uniform(sp + 1), begin_blk = ld_uniform(sp + 2),
            end_blk = ld_uniform(sp + 3), begin_piece = ld_uniform(sp + 4);

  const int rt0 = rg * NW;                  // first 32-row tile of this workgroup
  const int rt = rt0 + wave;                // the tile whose S^T / softmax this wave owns
  const int h = lane >> 5;                  // which half of the MFMA k / row slots
  const int col = lane & 31;                // MFMA column = query row within a tile
  const int r = rt * 32 + col;              // this lane's query row (as row owner)
  const bool row_ok = r < p.R;

  const unsigned lds0 = (unsigned)(size_t)(LDS_PTR(unsigned char))smem;
  LDS_PTR(unsigned char) lds = (LDS_PTR(unsigned char))smem;
  LDS_PTR(unsigned char) pb = (LDS_PTR(unsigned char))pbuf;
  const unsigned dma_off[2] = {dma_lane_offset(lane, 0), dma_lane_offset(lane, 1)};

  // QK^T A fragment of k-step ks, token tile tau: token col + 32 tau, logical
  // chunk 2 ks + h, i.e. block ks / 4, in-block chunk 2 (ks % 4) + h.
  const int qk_sw = chunk_xor(col);
  int qk_base[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) qk_base[b] = col * 128 + (((2 * b + h) ^ qk_sw) << 4);

  // Transposing V reads: 16-lane group G, lane Lq in it reads 8 bytes of
  // token 16 kk + 4 h + Lq / 4 (and + 8) at columns 32 ct + 16 (G & 1) + 4 (Lq & 3),
  // i.e. block ct / 2, in-block chunk 4 (ct % 2) + 2 (G & 1) + (Lq & 3) / 2.
  const int G = lane >> 4, Lq = lane & 15;
  const int rsub = 4 * (G >> 1) + (Lq >> 2);
  const int cc0 = 2 * (G & 1) + ((Lq & 3) >> 1);
  const int hb = (Lq & 1) * 8;
  int pv_base[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    pv_base[par][0] = rsub * 128 + (((4 * par + cc0) ^ chunk_xor(rsub)) << 4) + hb;
    pv_base[par][1] = (rsub + 8) * 128 + (((4 * par + cc0) ^ chunk_xor(rsub + 8)) << 4) + hb;
  }

  for (int req = begin_req; req <= end_req; ++req) {
    const int L = ld_uniform(p.seqlens + req);
    const int nblk = (L + kPage - 1) / kPage;
    const int lo = (req == begin_req) ? begin_blk : 0;
    const int hi = (req == end_req) ? end_blk : nblk;
    const int piece = (req == begin_req) ? begin_piece : 0;
    const int slot0 = ld_uniform(p.num_splits + req);
    const bool split = (ld_uniform(p.num_splits + req + 1) - slot0) > 1;
    const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;

    f32x16 o[NW][kCtPerWave];              // O^T tiles: all row tiles x this wave's columns
    bf16x8 qf[kKSteps];
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    for (int restarts = 0;; ++restarts) {
    if (lo < hi) issue_page<NW>(p.kv + (size_t)ld_uniform(bt + (lo)) * kPageBytes, lds0, dma_off, wave);
    // Q^T fragments (B operand): row r, dims 16 ks + 8 h .. + 7.
    {
      const unsigned char* qrow = p.q + ((size_t)req * p.R + (row_ok ? r : 0)) * kRowBytes + h * 16;
      const unsigned keep = row_ok ? ~0u : 0u;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        u32x4 v = *(const u32x4*)(qrow + ks * 32);
        v &= keep;
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    // Wait (visibly to the compiler) for Q and the first page, so that it
    // inserts no vmcnt(0) inside the page loop, where that would also wait
    // for the next page's copy.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int a = 0; a < NW; ++a)
#pragma unroll
      for (int c = 0; c < kCtPerWave; ++c) o[a][c] = f32x16{};
    l_run = 0.f;
    bool restart = false;

    for (int j = lo; j < hi; ++j) {
      const int bsel = (j - lo) & 1;
      LDS_PTR(unsigned char) buf = lds + bsel * kPageBytes;
      // Page j was copied while page j - 1 was computed (or in the prologue).
      wait_vmcnt<0>();
      lds_barrier();
      // The copy of page j + 1 into the other buffer (free since the end of
      // page j - 1) is interleaved with this page's QK^T MFMAs below.
      const bool has_next = j + 1 < hi;
      const unsigned char* next_page =
          uniform_ptr(p.kv + (size_t)ld_uniform(bt + (has_next ? j + 1 : j)) * kPageBytes);
      const unsigned next_lds = lds0 + (bsel ^ 1) * kPageBytes;
      const int valid = min(kPage, L - j * kPage);
      if (valid < kPage) {
        // Tokens past the sequence end: zero their rows in every column block
        // so that masked probabilities (exactly 0) never meet non-finite
        // cache contents.
        const int per_blk = (kPage - valid) * 8;
        for (int u = threadIdx.x; u < per_blk * 9; u += NW * 64) {
          const int b = u / per_blk, w = u - b * per_blk;
          *(LDS_PTR(u32x4))(buf + b * kBlockBytes + valid * 128 + w * 16) = u32x4{0, 0, 0, 0};
        }
        lds_barrier();
      }

      // ---- S^T = K Q^T for this wave's row tile, one 32-token tile at a time
      // (tokens 0..31, then 32..63), each followed by its softmax and the
      // write of its bf16 P fragments; K fragments are read one k-step ahead.
      // The piece's reference max comes from the first token tile.  Lane
      // holds tokens 32 tile + 8 (v / 4) + 4 h + v % 4 of row col.
      const bool tail = valid < kPage;
      bool wave_bad = false;
      float lsum = 0.f;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        f32x16 sacc = f32x16{};
        {
          auto kfrag = [&](int ks) -> bf16x8 {
            LDS_PTR(unsigned char) a = buf + (ks >> 2) * kBlockBytes + qk_base[ks & 3] + tile * 32 * 128;
            return __builtin_bit_cast(bf16x8, *(LDS_PTR(u32x4))(a));
          };
          bf16x8 k0 = kfrag(0), k1 = kfrag(1);
          constexpr int kPerTile = kSlices / NW / 2;            // DMA slices per token tile
          constexpr int kStride = kKSteps / kPerTile;           // MFMAs between slices
#pragma unroll
          for (int ks = 0; ks < kKSteps; ++ks) {
            bf16x8 n = k1;
            if (ks + 2 < kKSteps) n = kfrag(ks + 2);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], sacc, 0, 0, 0);
            if (has_next && ks % kStride == kStride - 1 && ks / kStride < kPerTile)
              issue_slice<NW>(next_page, next_lds, dma_off, wave, tile * kPerTile + ks / kStride);
            k0 = k1;
            k1 = n;
          }
        }
        // (softmax_scale >= 0, so the max of the raw scores, scaled, is the
        // max of the scaled scores; masked tokens are left out of the max and
        // get probability exactly 0.)
        float mloc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tok = 32 * tile + 8 * (v >> 2) + 4 * h + (v & 3);
          mloc = fmaxf(mloc, (tail && tok >= valid) ? -INFINITY : sacc[v]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * p.scale_log2;
        m_seen = fmaxf(m_seen, mloc);
        if (j == lo && restarts == 0 && tile == 0) m_ref = mloc;
        wave_bad |= __any(mloc > m_ref + kRefHeadroom) && restarts < kMaxRestarts;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int kk = 2 * tile + half;   // 16-token k-step of the PV product
          bf16x8 pk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int v = 8 * half + e;
            const int tok = 32 * tile + 8 * (v >> 2) + 4 * h + (v & 3);
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], p.scale_log2, -m_ref));
            if (tail && tok >= valid) pe = 0.f;
            lsum += pe;   // row sum from the fp32 values; only the PV operand is bf16
            pk[e] = (__bf16)pe;
          }
          u32x4 bits = __builtin_bit_cast(u32x4, pk);
          if (kk == 3 && lane == 0)   // probabilities are >= 0: the sign bit carries the restart flag
            bits[0] = wave_bad ? (bits[0] | 0x8000u) : (bits[0] & ~0x8000u);
          *(LDS_PTR(u32x4))(pb + ((wave * 4 + kk) * 64 + lane) * 16) = bits;
        }
      }
      l_run += lsum;
      lds_barrier();  // every wave's P is in LDS

      int any_bad = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        any_bad |= *(LDS_PTR(unsigned short))(pb + ((w * 4 + 3) * 64) * 16) >> 15;
      if (any_bad && restarts < kMaxRestarts) {
        // Slow path: a row outgrew its reference max.  Drain the copy in
        // flight, then redo the piece from its first page with the largest
        // max seen so far as the reference.
        wait_vmcnt<0>();
        lds_barrier();
        restart = true;
        break;
      }

      // ---- O^T += V^T P^T: this wave's columns, every row tile of the group.
      {
        auto vfrag = [&](int kk, int ct) -> bf16x8 {
          LDS_PTR(unsigned char) a = buf + (ct >> 1) * kBlockBytes + kk * 16 * 128;
          const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_base[ct & 1][0]));
          const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_base[ct & 1][1]));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        const int ct0 = wave * kCtPerWave;
        bf16x8 vcur = vfrag(0, ct0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          bf16x8 pf[NW];
#pragma unroll
          for (int a = 0; a < NW; ++a)
            pf[a] = __builtin_bit_cast(bf16x8, *(LDS_PTR(u32x4))(pb + ((a * 4 + kk) * 64 + lane) * 16));
#pragma unroll
          for (int c = 0; c < kCtPerWave; ++c) {
            bf16x8 vnext = vcur;
            if (c + 1 < kCtPerWave) vnext = vfrag(kk, ct0 + c + 1);
            else if (kk + 1 < 4) vnext = vfrag(kk + 1, ct0);
#pragma unroll
            for (int a = 0; a < NW; ++a)
              o[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pf[a], o[a][c], 0, 0, 0);
            vcur = vnext;
          }
        }
      }

      lds_barrier();  // every wave is done with this page buffer and with P
    }
    if (!restart) break;
    m_ref = m_seen;
    }

    // ---- epilogue.  Row owners publish 1 / l for their rows through LDS
    // (the P buffer is free after the last page's barrier); every wave then
    // normalises its columns for all row tiles of the group.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    if (h == 0) *(LDS_PTR(float))(pb + (wave * 32 + col) * 4) = inv;
    lds_barrier();
    float inv_rows[NW];
#pragma unroll
    for (int a = 0; a < NW; ++a) inv_rows[a] = *(LDS_PTR(float))(pb + (a * 32 + col) * 4);
    lds_barrier();  // the next piece's first P writes come after this
    if (!split) {
#pragma unroll
      for (int a = 0; a < NW; ++a) {
        const int ra = (rt0 + a) * 32 + col;
        if (ra >= p.R) continue;
        unsigned short* orow = p.out + ((size_t)req * p.R + ra) * kDv;
#pragma unroll
        for (int c = 0; c < kCtPerWave; ++c) {
          const int ct = wave * kCtPerWave + c;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 w4;
#pragma unroll
            for (int e = 0; e < 4; ++e) w4[e] = (__bf16)(o[a][c][4 * g + e] * inv_rows[a]);
            *(bf16x4*)(orow + 32 * ct + 8 * g + 4 * h) = w4;
          }
        }
      }
      if (h == 0 && row_ok) {
        const int s = r / p.h_q, hh = r - s * p.h_q;
        p.lse[((size_t)req * p.h_q + hh) * p.s_q + s] = lse2 * kLn2;
      }
    } else {
      const int slot = slot0 + piece;
#pragma unroll
      for (int a = 0; a < NW; ++a) {
        if (rt0 + a >= p.row_tiles) continue;
        float* dst = p.oacc + ((((size_t)slot * p.row_tiles + rt0 + a) * kColTiles) * 64 + lane) * 16;
#pragma unroll
        for (int c = 0; c < kCtPerWave; ++c) {
          const int ct = wave * kCtPerWave + c;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 w4;
#pragma unroll
            for (int e = 0; e < 4; ++e) w4[e] = o[a][c][4 * g + e] * inv_rows[a];
            *(f32x4*)(dst + (size_t)ct * 64 * 16 + 4 * g) = w4;
          }
        }
      }
      if (h == 0 && rt < p.row_tiles) p.lacc[(size_t)slot * p.row_tiles * 32 + r] = lse2;
    }
  }
}

// Small row counts (R = s_q * h_q <= 16), the memory-bound regime.  Wave w
// owns tokens 16 w .. 16 w + 15 of every page of the piece and runs its own
// pipeline: it copies just those 16 token rows (18 KiB) into a private pair
// of LDS stages, so the page loop has no workgroup barrier at all, and each
// wave keeps its own softmax state, merged with the other three through LDS
// when the piece ends (log-sum-exp rule).
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of
//     K (one ds_read_b128 per lane), B = Q^T held in registers.
//   * The S^T accumulator (lane = query row, 4 consecutive tokens) is the B
//     operand of v_mfma_f32_16x16x16_bf16 for O^T = V^T P^T; V^T fragments
//     (4 consecutive tokens of one column) come from ds_read_b64_tr_b16.
//   * Probabilities use a fixed per-wave reference: the wave's row max over
//     its first page.  If a later score exceeds it by more than 2^64 the wave
//     redoes the piece once with the exact maximum as the reference, so the
//     accumulator is never rescaled and stays in AGPRs.
constexpr int kWaveTokens = 16;
constexpr int kStageBytes = kWaveTokens * kRowBytes;   // 18 KiB: 16 token rows
constexpr int kStageSlices = kStageBytes / 1024;       // 18 wave-wide 1 KiB copies
constexpr int kStageBlock = kWaveTokens * 128;         // one 64-dim column block of a stage

// Chunk position of logical chunk c of local token t (0..15) in a stage is
// c ^ stage_swizzle(t): 16 tokens at one chunk (the QK read) and 8 tokens x a
// chunk pair (the transposing PV read, 32 lanes) both land on distinct banks.
__device__ __forceinline__ int stage_swizzle(int t) { return 2 * ((t >> 1) & 3) + ((t >> 3) & 1); }

// Global byte offset of lane `lane`'s 16 bytes within slice parity `par` of a
// wave's 16-token row group: local token 8 par + lane / 8, chunk position lane % 8.
__device__ __forceinline__ unsigned stage_dma_offset(int lane, int par) {
  const int t = 8 * par + (lane >> 3);
  return (unsigned)(t * kRowBytes + (((lane & 7) ^ stage_swizzle(t)) << 4));
}

// Copy slice i (block i / 2, tokens 8 (i % 2) .. + 7) of this wave's rows.
__device__ __forceinline__ void issue_stage_slice(const unsigned char* rows, unsigned stage_lds,
                                                  const unsigned dma_off[2], int i) {
  unsigned lane_off = dma_off[i & 1];
  asm volatile("" : "+v"(lane_off));
  const unsigned voff = lane_off + (unsigned)((i >> 1) * 128);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(stage_lds + (unsigned)i * 1024u);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(rows), "s"(m0)
               : "memory");
}

__global__ void __launch_bounds__(256, 1) mla_splitkv_small_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * 2 * kStageBytes];
  __shared__ float st_m[4][16], st_l[4][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = blockIdx.x;
  if (part >= p.num_parts) return;
  const int32_t* sp = p.sched + part * MLA_SCHED_INTS;
  const int begin_req = ld_uniform(sp), end_req = ld_uniform(sp + 1), begin_blk = ld_uniform(sp + 2),
            end_blk = ld_uniform(sp + 3), begin_piece = ld_uniform(sp + 4);

  const int g = lane >> 4;     // 16-lane group
  const int c16 = lane & 15;   // MFMA column = query row
  const bool row_ok = c16 < p.R;
  const int tok0 = kWaveTokens * wave;

  LDS_PTR(unsigned char) wlds = (LDS_PTR(unsigned char))smem + wave * 2 * kStageBytes;
  const unsigned wlds0 = (unsigned)(size_t)wlds;
  const unsigned dma_off[2] = {stage_dma_offset(lane, 0), stage_dma_offset(lane, 1)};

  // QK A fragment of k-step ks: local token c16, logical chunk 4 ks + g =
  // block ks / 2, in-block chunk 4 (ks % 2) + g.
  int qk_off[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) qk_off[b] = c16 * 128 + (((4 * b + g) ^ stage_swizzle(c16)) << 4);
  // PV A fragment of column tile ct: lane (group g, index c16) reads local
  // token 4 g + c16 / 4, columns 16 ct + 4 (c16 % 4) .. + 3 = block ct / 4,
  // in-block chunk 2 (ct % 4) + (c16 % 4) / 2, byte 8 (c16 % 2).
  const int tv = 4 * g + (c16 >> 2);
  int pv_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    pv_off[m] = tv * 128 + (((2 * m + ((c16 & 3) >> 1)) ^ stage_swizzle(tv)) << 4) + (c16 & 1) * 8;

  for (int req = begin_req; req <= end_req; ++req) {
    const int L = ld_uniform(p.seqlens + req);
    const int nblk = (L + kPage - 1) / kPage;
    const int lo = (req == begin_req) ? begin_blk : 0;
    const int hi = (req == end_req) ? end_blk : nblk;
    const int piece = (req == begin_req) ? begin_piece : 0;
    const int slot0 = ld_uniform(p.num_splits + req);
    const bool split = (ld_uniform(p.num_splits + req + 1) - slot0) > 1;
    const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;
    auto rows_of = [&](int j) {
      return uniform_ptr(p.kv + (size_t)ld_uniform(bt + j) * kPageBytes + (size_t)tok0 * kRowBytes);
    };

    f32x4 o[kDv / 16];
    float m_ref = -INFINITY, l_run = 0.f;
    bool have_ref = false;
    for (int attempt = 0;; ++attempt) {
      if (lo < hi) {
        const unsigned char* r0 = rows_of(lo);
#pragma unroll
        for (int i = 0; i < kStageSlices; ++i) issue_stage_slice(r0, wlds0, dma_off, i);
      }
      // Q^T fragments (B operand): row c16, dims 32 ks + 8 g .. + 7.
      bf16x8 qf[kDqk / 32];
      {
        const unsigned char* qrow = p.q + ((size_t)req * p.R + (row_ok ? c16 : 0)) * kRowBytes + g * 16;
        const unsigned keep = row_ok ? ~0u : 0u;
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks) {
          u32x4 v = *(const u32x4*)(qrow + ks * 64);
          v &= keep;
          qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
      }
      // Q and the first page (compiler-visible, so the page loop only ever
      // waits on the copies it issues itself); the second page's copy then
      // overlaps the first page's arithmetic.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      if (lo + 1 < hi) {
        const unsigned char* r1 = rows_of(lo + 1);
#pragma unroll
        for (int i = 0; i < kStageSlices; ++i) issue_stage_slice(r1, wlds0 + kStageBytes, dma_off, i);
      }

#pragma unroll
      for (int ct = 0; ct < kDv / 16; ++ct) o[ct] = f32x4{0, 0, 0, 0};
      float m_seen = -INFINITY;
      l_run = 0.f;

      for (int j = lo; j < hi; ++j) {
        const int stage = (j - lo) & 1;
        LDS_PTR(unsigned char) buf = wlds + stage * kStageBytes;
        if (j + 1 < hi)
          wait_vmcnt<kStageSlices>();
        else
          wait_vmcnt<0>();
        const int valid = min(kPage, L - j * kPage) - tok0;   // valid local tokens (may be <= 0)
        if (valid < kWaveTokens) {
          // Zero the V part of this wave's rows past the end of the sequence
          // (page tails may hold anything, NaN included; P is 0 there).
          const int t_first = max(valid, 0);
          const int n = (kWaveTokens - t_first) * 8 * 8;      // 16-byte chunks in blocks 0..7
          for (int u = lane; u < n; u += 64) {
            const int t = t_first + (u >> 6), b = (u >> 3) & 7, c = u & 7;
            *(LDS_PTR(u32x4))(buf + b * kStageBlock + t * 128 + c * 16) = u32x4{0, 0, 0, 0};
          }
        }

        // ---- S^T (16 tokens x 16 rows) = K Q^T, three accumulation chains.
        u32x4 kf[kDqk / 32];
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks)
          kf[ks] = *(LDS_PTR(u32x4))(buf + (ks >> 1) * kStageBlock + qk_off[ks & 1]);
        f32x4 sacc[3] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
        for (int ks = 0; ks < kDqk / 32; ++ks)
          sacc[ks % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks],
                                                                  sacc[ks % 3], 0, 0, 0);
        const f32x4 sv = sacc[0] + sacc[1] + sacc[2];

        // ---- probabilities against the fixed reference (base 2).
        float x[4];
        float mloc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[v] = (4 * g + v) < valid ? sv[v] * p.scale_log2 : -INFINITY;
          mloc = fmaxf(mloc, x[v]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        if (!have_ref) m_ref = mloc;   // first page of the first attempt
        have_ref = true;
        m_seen = fmaxf(m_seen, mloc);
        i16x4 pb;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float pe = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[v] - m_ref);
          l_run += pe;
          pb[v] = __builtin_bit_cast(short, (__bf16)pe);
        }

        // ---- O^T (512 x 16) += V^T (512 x 16 tokens) P^T, two batches of reads.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          i16x4 vf[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const int ct = 16 * h + k;
            vf[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_PTR(i16x4))(buf + (ct >> 2) * kStageBlock + pv_off[ct & 3]));
          }
          if (h == 1) {
            // Every read of this stage has been issued; once they complete the
            // stage takes page j + 2.
            if (j + 2 < hi) {
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              const unsigned char* r2 = rows_of(j + 2);
#pragma unroll
              for (int i = 0; i < kStageSlices; ++i)
                issue_stage_slice(r2, wlds0 + stage * kStageBytes, dma_off, i);
            }
          }
#pragma unroll
          for (int k = 0; k < 16; ++k)
            o[16 * h + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[k], pb, o[16 * h + k], 0, 0, 0);
        }
      }
      // One retry with the exact maximum always suffices: every probability is then <= 1.
      if (attempt > 0 || !__any(m_seen > m_ref + kRefHeadroom)) break;
      m_ref = m_seen;
    }

    // ---- merge the four waves' states.  Each wave parks its accumulator in
    // its own stages (its copies are all complete), then every wave
    // finalises 128 of the 512 columns.
    float lw = l_run + __shfl_xor(l_run, 16);
    lw += __shfl_xor(lw, 32);
    if (g == 0) {
      st_m[wave][c16] = m_ref;
      st_l[wave][c16] = lw;
    }
#pragma unroll
    for (int ct = 0; ct < kDv / 16; ++ct) *(LDS_PTR(f32x4))(wlds + (ct * 64 + lane) * 16) = o[ct];
    lds_barrier();
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (st_l[w][c16] > 0.f) M = fmaxf(M, st_m[w][c16]);
    float wgt[4], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wgt[w] = st_l[w][c16] > 0.f ? __builtin_amdgcn_exp2f(st_m[w][c16] - M) : 0.f;
      lsum += wgt[w] * st_l[w][c16];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? M + __builtin_amdgcn_logf(lsum) : -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int ct = 8 * wave + k;
      f32x4 acc = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 4; ++w)
        acc += wgt[w] * *(LDS_PTR(f32x4))((LDS_PTR(unsigned char))smem + w * 2 * kStageBytes + (ct * 64 + lane) * 16);
      acc *= inv;
      if (!row_ok) continue;
      const int c = 16 * ct + 4 * g;   // 4 consecutive columns of row c16
      if (!split) {
        bf16x4 w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = (__bf16)acc[e];
        *(bf16x4*)(p.out + ((size_t)req * p.R + c16) * kDv + c) = w4;
      } else {
        // Partial slot in the 32-row-tile layout the combine kernel reads:
        // [slot][row tile 0][c / 32][lane32][16], lane32 = row + 32 ((c % 32) / 4 % 2),
        // element 4 ((c % 32) / 8) + c % 4.
        const int cc = c & 31;
        const int lane32 = c16 + 32 * ((cc >> 2) & 1);
        float* dst = p.oacc + ((((size_t)(slot0 + piece) * p.row_tiles) * kColTiles + (c >> 5)) * 64 + lane32) * 16 +
                     4 * (cc >> 3);
        *(f32x4*)dst = acc;
      }
    }
    if (wave == 0 && g == 0 && row_ok) {
      if (!split) {
        const int s = c16 / p.h_q, hh = c16 - s * p.h_q;
        p.lse[((size_t)req * p.h_q + hh) * p.s_q + s] = lse2 * kLn2;
      } else {
        p.lacc[(size_t)(slot0 + piece) * p.row_tiles * 32 + c16] = lse2;
      }
    }
    lds_barrier();  // every wave is done reading the parked accumulators
  }
}

// Merge the partial (O_i, lse_i) of every split request (the log-sum-exp
// merge of the attention-kernel page and the overview page, section 7):
// M = max lse_i, w_i = 2^(lse_i - M), out = sum w_i O_i / sum w_i,
// lse = M + log2(sum w_i) (then converted to natural log).  One workgroup per
// (request, 32-row tile, 32-column tile); lane = accumulator lane of the main
// kernel, so every partial read is a contiguous 64-byte run per lane.  The
// four waves take every fourth split, two in flight at a time, and are
// summed through LDS.
constexpr int kCombineWaves = 4;

__global__ void __launch_bounds__(kCombineWaves * 64) mla_combine_kernel(Params p) {
  __shared__ float red_max[kCombineWaves][64];
  __shared__ f32x4 red_acc[kCombineWaves - 1][4][64];
  __shared__ float red_w[kCombineWaves - 1][64];
  const int per_req = p.row_tiles * kColTiles;
  const int req = blockIdx.x / per_req;
  const int rem = blockIdx.x - req * per_req;
  const int rt = rem / kColTiles, ct = rem - rt * kColTiles;
  const int slot0 = ld_uniform(p.num_splits + req);
  const int n = ld_uniform(p.num_splits + req + 1) - slot0;
  if (n <= 1) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int r = rt * 32 + (lane & 31);
  const size_t rows_p = (size_t)p.row_tiles * 32;
  const float* lrow = p.lacc + (size_t)slot0 * rows_p + r;
  const size_t ostride = (size_t)p.row_tiles * kColTiles * 64 * 16;   // floats per slot
  const float* obase = p.oacc + ((((size_t)slot0 * p.row_tiles + rt) * kColTiles + ct) * 64 + lane) * 16;

  float M = -INFINITY;
  for (int i = wave; i < n; i += kCombineWaves) M = fmaxf(M, lrow[(size_t)i * rows_p]);
  red_max[wave][lane] = M;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) M = fmaxf(M, red_max[w][lane]);

  f32x4 acc[4] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  float wsum = 0.f;
  if (M != -INFINITY) {
    int i = wave;
    for (; i + kCombineWaves < n; i += 2 * kCombineWaves) {
      const int i2 = i + kCombineWaves;
      const float l1 = lrow[(size_t)i * rows_p], l2 = lrow[(size_t)i2 * rows_p];
      const f32x4* s1 = (const f32x4*)(obase + (size_t)i * ostride);
      const f32x4* s2 = (const f32x4*)(obase + (size_t)i2 * ostride);
      const f32x4 a0 = s1[0], a1 = s1[1], a2 = s1[2], a3 = s1[3];
      const f32x4 b0 = s2[0], b1 = s2[1], b2 = s2[2], b3 = s2[3];
      const float w1 = __builtin_amdgcn_exp2f(l1 - M), w2 = __builtin_amdgcn_exp2f(l2 - M);
      wsum += w1 + w2;
      acc[0] += w1 * a0 + w2 * b0;
      acc[1] += w1 * a1 + w2 * b1;
      acc[2] += w1 * a2 + w2 * b2;
      acc[3] += w1 * a3 + w2 * b3;
    }
    if (i < n) {
      const float w1 = __builtin_amdgcn_exp2f(lrow[(size_t)i * rows_p] - M);
      const f32x4* s1 = (const f32x4*)(obase + (size_t)i * ostride);
      wsum += w1;
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] += w1 * s1[g];
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) red_acc[wave - 1][g][lane] = acc[g];
    red_w[wave - 1][lane] = wsum;
  }
  __syncthreads();
  if (wave > 0 || r >= p.R) return;
#pragma unroll
  for (int w = 0; w < kCombineWaves - 1; ++w) {
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] += red_acc[w][g][lane];
    wsum += red_w[w][lane];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  unsigned short* orow = p.out + ((size_t)req * p.R + r) * kDv;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2 w;
    w[0] = (unsigned)f32_to_bf16(acc[g][0] * inv) | ((unsigned)f32_to_bf16(acc[g][1] * inv) << 16);
    w[1] = (unsigned)f32_to_bf16(acc[g][2] * inv) | ((unsigned)f32_to_bf16(acc[g][3] * inv) << 16);
    *(u32x2*)(orow + 32 * ct + 8 * g + 4 * h) = w;
  }
  if (ct == 0 && h == 0) {
    const int s = r / p.h_q, hh = r - s * p.h_q;
    p.lse[((size_t)req * p.h_q + hh) * p.s_q + s] =
        (M == -INFINITY || !(wsum > 0.f)) ? -INFINITY : (M + __builtin_amdgcn_logf(wsum)) * kLn2;
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" const char* mla_last_error(void) { return g_last_error.c_str(); }

extern "C" int mla_plan(const int32_t* cache_seqlens, int batch, int num_parts, int fixed_overhead,
                        int force_splits, int32_t* sched_out, int max_parts, int32_t* num_splits_out,
                        int* num_parts_out) {
  return plan(cache_seqlens, batch, num_parts, fixed_overhead, force_splits, sched_out, max_parts,
              num_splits_out, num_parts_out);
}

static int policy(const int32_t* seqlens, int batch, int h_q, int s_q, int* num_cus, int* parts, int* F) {
  if (batch <= 0 || h_q <= 0 || s_q <= 0 || !seqlens)
    return set_error(MLA_ERR_INVALID, "mla_get_metadata: batch=%d h_q=%d s_q=%d seqlens=%p", batch, h_q, s_q,
                     (const void*)seqlens);
  if (*num_cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return set_error(MLA_ERR_HIP, "mla_get_metadata: cannot query the CU count");
  }
  const Geometry g = geometry(h_q, s_q);
  *parts = *num_cus / g.row_groups;
  if (*parts < 1) *parts = 1;
  *F = g.R <= 32 ? 1 : 2;
  return MLA_OK;
}

extern "C" int mla_max_parts(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int num_cus,
                             int force_splits) {
  int parts, F;
  int rc = policy(cache_seqlens, batch, h_q, s_q, &num_cus, &parts, &F);
  if (rc) return rc;
  if (force_splits <= 0) return parts;
  long long total = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = (cache_seqlens[b] + kPage - 1) / kPage;
    total += n < 1 ? 1 : (n < force_splits ? n : force_splits);
  }
  return (int)total;
}

extern "C" int mla_get_metadata(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int num_cus,
                                int force_splits, int32_t* sched_out, int max_parts,
                                int32_t* num_splits_out, int* num_parts_out, int* total_splits_out) {
  int parts, F;
  int rc = policy(cache_seqlens, batch, h_q, s_q, &num_cus, &parts, &F);
  if (rc) return rc;
  if (!total_splits_out) return set_error(MLA_ERR_INVALID, "mla_get_metadata: null total_splits_out");
  rc = plan(cache_seqlens, batch, parts, F, force_splits, sched_out, max_parts, num_splits_out, num_parts_out);
  if (rc) return rc;
  *total_splits_out = num_splits_out[batch];
  return MLA_OK;
}

extern "C" size_t mla_workspace_bytes(int total_splits, int h_q, int s_q) {
  if (total_splits <= 0 || h_q <= 0 || s_q <= 0) return 0;
  const Geometry g = geometry(h_q, s_q);
  const size_t rows = (size_t)total_splits * g.row_tiles * 32;
  return align256(rows * kDv * sizeof(float)) + align256(rows * sizeof(float));
}

// Event recording for mla_profile_start / mla_profile_stop (benchmarks only).
namespace mla {
namespace {
struct Profile {
  bool on = false;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev;  // 3 per call: before main, after main, after combine
};
Profile g_prof;
std::mutex g_prof_mu;
}  // namespace
}  // namespace mla

extern "C" int mla_profile_start(int max_calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (max_calls <= 0 || g_prof.on) return set_error(MLA_ERR_INVALID, "mla_profile_start: max_calls=%d on=%d", max_calls, (int)g_prof.on);
  g_prof.ev.assign((size_t)max_calls * 3, nullptr);
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return set_error(MLA_ERR_HIP, "mla_profile_start: hipEventCreate failed");
  g_prof.cap = max_calls;
  g_prof.used = 0;
  g_prof.on = true;
  return MLA_OK;
}

extern "C" int mla_profile_stop(float* main_ms, float* combine_ms, int* calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on || !main_ms || !combine_ms || !calls) return set_error(MLA_ERR_INVALID, "mla_profile_stop: not started or null output");
  float a = 0.f, c = 0.f;
  int rc = MLA_OK;
  if (g_prof.used > 0 && hipEventSynchronize(g_prof.ev[(size_t)g_prof.used * 3 - 1]) != hipSuccess)
    rc = set_error(MLA_ERR_HIP, "mla_profile_stop: hipEventSynchronize failed");
  for (int i = 0; rc == MLA_OK && i < g_prof.used; ++i) {
    float t0 = 0.f, t1 = 0.f;
    if (hipEventElapsedTime(&t0, g_prof.ev[i * 3], g_prof.ev[i * 3 + 1]) != hipSuccess ||
        hipEventElapsedTime(&t1, g_prof.ev[i * 3 + 1], g_prof.ev[i * 3 + 2]) != hipSuccess)
      rc = set_error(MLA_ERR_HIP, "mla_profile_stop: hipEventElapsedTime failed");
    a += t0;
    c += t1;
  }
  *main_ms = a;
  *combine_ms = c;
  *calls = g_prof.used;
  for (auto e : g_prof.ev) hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on = false;
  return rc;
}

static hipEvent_t* profile_slot() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on || g_prof.used >= g_prof.cap) return nullptr;
  return &g_prof.ev[(size_t)(g_prof.used++) * 3];
}

extern "C" int mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_blocks,
                              int max_blocks_per_seq, float softmax_scale, const int32_t* sched,
                              int num_parts, const int32_t* num_splits, void* workspace,
                              size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !sched || !num_splits || !out || !lse)
    return set_error(MLA_ERR_INVALID, "mla_decode_fwd: null pointer argument");
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || num_parts <= 0)
    return set_error(MLA_ERR_INVALID,
                     "mla_decode_fwd: batch=%d s_q=%d h_q=%d num_blocks=%d max_blocks_per_seq=%d num_parts=%d",
                     batch, s_q, h_q, num_blocks, max_blocks_per_seq, num_parts);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return set_error(MLA_ERR_INVALID, "mla_decode_fwd: softmax_scale must be finite and >= 0");
  const Geometry g = geometry(h_q, s_q);
  const int slots = num_parts + batch - 1;
  const size_t need = mla_workspace_bytes(slots, h_q, s_q);
  if (!workspace || workspace_bytes < need)
    return set_error(MLA_ERR_WORKSPACE, "mla_decode_fwd: workspace %zu bytes < %zu needed", workspace_bytes, need);

  Params prm;
  prm.q = (const unsigned char*)q;
  prm.kv = (const unsigned char*)kv_cache;
  prm.block_table = block_table;
  prm.seqlens = cache_seqlens;
  prm.sched = sched;
  prm.num_splits = num_splits;
  prm.out = (unsigned short*)out;
  prm.lse = lse;
  const size_t rows = (size_t)slots * g.row_tiles * 32;
  prm.oacc = (float*)workspace;
  prm.lacc = (float*)((char*)workspace + align256(rows * kDv * sizeof(float)));
  prm.R = g.R;
  prm.h_q = h_q;
  prm.s_q = s_q;
  prm.max_blocks = max_blocks_per_seq;
  prm.num_parts = num_parts;
  prm.row_groups = g.row_groups;
  prm.row_tiles = g.row_tiles;
  prm.scale_log2 = softmax_scale * kLog2e;

  hipStream_t st = (hipStream_t)stream;
  hipEvent_t* ev = profile_slot();
  if (ev) hipEventRecord(ev[0], st);
  const int grid = g.row_groups == 1 ? num_parts : 8 * g.row_groups * ((num_parts + 7) / 8);
  if (g.R <= 16) {
    hipLaunchKernelGGL(mla_splitkv_small_kernel, dim3(num_parts), dim3(256), 0, st, prm);
  } else switch (g.waves) {
    case 1: hipLaunchKernelGGL(mla_splitkv_kernel<1>, dim3(grid), dim3(64), 0, st, prm); break;
    case 2: hipLaunchKernelGGL(mla_splitkv_kernel<2>, dim3(grid), dim3(128), 0, st, prm); break;
    case 4: hipLaunchKernelGGL(mla_splitkv_kernel<4>, dim3(grid), dim3(256), 0, st, prm); break;
    default: return set_error(MLA_ERR_INVALID, "mla_decode_fwd: unsupported wave count %d", g.waves);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "mla_decode_fwd: main kernel launch: %s", hipGetErrorString(e));
  if (ev) hipEventRecord(ev[1], st);
  hipLaunchKernelGGL(mla_combine_kernel, dim3(batch * g.row_tiles * kColTiles), dim3(kCombineWaves * 64), 0, st, prm);
  e = hipGetLastError();
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "mla_decode_fwd: combine launch: %s", hipGetErrorString(e));
  if (ev) hipEventRecord(ev[2], st);
  return MLA_OK;
}
