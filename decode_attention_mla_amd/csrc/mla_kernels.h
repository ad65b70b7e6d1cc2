// Device code of the MLA decode library for MI355X (gfx950): the split-KV
// kernels, the log-sum-exp combine kernel, the device planner and their
// device helpers.  Included once, by mla_decode.hip (the C ABI and the
// launches), which must see the kernels' definitions to launch them.
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
//   * Every split-KV workgroup has four waves, one per SIMD, and wave w
//     copies tokens 16 w .. 16 w + 15 of every page (18 KiB) into LDS with
//     global_load_lds_dwordx4 (16 B per lane straight into LDS), issued a
//     page ahead and spread between the MFMAs.  Three kernels by row count
//     R = s_q * h_q:
//       - R <= 16 (memory-bound decode): one workgroup per part; the four
//         slices form a shared page stage (two stages), a barrier makes a
//         page visible; QK^T split by tokens (v_mfma_f32_16x16x32_bf16),
//         probabilities exchanged through LDS, PV split by columns.
//       - 16 < R < 128 (bf16 cache only): one workgroup per 32 rows; each
//         wave keeps private stages and its own softmax state over its
//         tokens, with no barrier in the page loop; the four states are
//         merged through LDS when a piece ends.
//       - R >= 128 (and sparse or FP8 above 16 rows): one workgroup per 128
//         rows; shared stages; QK^T split by rows
//         (v_mfma_f32_32x32x16_bf16, Q^T in registers), probabilities
//         exchanged through LDS, PV split by columns with O^T in AGPRs.
//   * In LDS a 16-token slice holds nine 64-dim column blocks; block b has
//     one 128-byte row per token whose eight 16-byte chunks are permuted by a
//     function of the token, so that the row reads of QK^T and the
//     transposing reads of PV (ds_read_b64_tr_b16) spread over the banks.
//   * Softmax runs in base 2 with log2(e) folded into the score scale (the
//     exp2 detail of the FlashMLA new-kernel deep-dive page).  Instead of
//     moving the running max every page and rescaling O (which would drag the
//     accumulator through VALU each page), a piece keeps the row max of the
//     first page in which a row sees a key as a fixed reference:
//     probabilities are 2^(s - m_ref) and may exceed 1.  This is the
//     online-softmax algebra with a fixed reference, exact up to rounding.  If
//     a row's max ever rises more than 64 (log2) above its reference, the
//     workgroup redoes the piece once with the exact maxima as references, so
//     nothing can overflow.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kRowBytes = kDqk * 2;                // 1152
constexpr int kPageBytes = kPage * kRowBytes;      // 73728
constexpr int kQkSteps = kDqk / 32;                // 18 k-steps of 32 dims (16x16x32 MFMA)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefHeadroom = 64.0f;              // log2 units a row max may exceed its reference

struct Params {
  const unsigned char* q;      // bf16 [batch, R, 576]
  const unsigned char* kv;     // bf16 [num_blocks, 64, 576]
  const int32_t* block_table;  // [batch, max_blocks]
  const int32_t* seqlens;      // [batch]
  const int32_t* sched;        // [num_parts, 8]
  const int32_t* num_splits;   // [batch + 1] exclusive prefix
  unsigned short* out;         // bf16 [batch, R, 512]
  float* lse;                  // [batch, h_q, s_q]
  float* oacc;                 // [slots, R, 512] normalised partial O
  float* lacc;                 // [slots, R] partial lse, base 2
  int batch, R, h_q, s_q, max_blocks, num_parts, row_groups;
  int causal;                  // 1: query token s of s_q sees keys 0 .. L - s_q + s
  float scale_log2;            // softmax_scale * log2(e)
  // Sparse decode (indices != nullptr): "request" v = b * fold + s is query
  // token s of request b, with R = h_q rows and s_q = 1 here; fold is the
  // real s_q (1 for dense decode), used to place lse.
  const int32_t* indices;      // [batch * fold, topk]: page_id * 64 + offset
  const int32_t* topk_len;     // [real batch]: entries of each list that count, or nullptr (all topk)
  int topk, kv_tokens, fold;
  // Small-row kernel: split partials go out with the nontemporal hint (1) or
  // as plain stores (0), chosen by the launch from the partials' size.
  int nt_partials;
};

// Keys query row `row` (= s * h_q + h) sees in a request of length L: all L,
// or with the causal mask of multi-token prediction the first
// L - (s_q - 1 - s) (the s_q query tokens are the sequence's last positions;
// the pages' is_causal flag).  May be <= 0.
__device__ __forceinline__ int row_keys(const Params& p, int L, int row) {
  return p.causal ? L - (p.s_q - 1 - row / p.h_q) : L;
}

// The arguments a workgroup needs before its first copy come first in
// every split-KV kernel's signature, as plain scalars, so that the
// dispatcher preloads them into SGPRs (built with kernel-argument
// preloading): no round trip to the argument segment precedes the read of
// the plan row.  The rest of Params is read from the argument segment as
// usual.  (The combine kernel has its own short list.)
#define MLA_SPLITKV_HOT_ARGS                                                                                  \
  const int32_t *hot_sched, int hot_num_parts, int hot_row_groups, int hot_max_blocks,                       \
      const int32_t *hot_block_table, const int32_t *hot_seqlens, const int32_t *hot_num_splits,              \
      const unsigned char *hot_kv, const unsigned char *hot_q
__device__ __forceinline__ Params with_hot_args(Params p, MLA_SPLITKV_HOT_ARGS) {
  p.sched = hot_sched;
  p.num_parts = hot_num_parts;
  p.row_groups = hot_row_groups;
  p.max_blocks = hot_max_blocks;
  p.block_table = hot_block_table;
  p.seqlens = hot_seqlens;
  p.num_splits = hot_num_splits;
  p.kv = hot_kv;
  p.q = hot_q;
  return p;
}
#define MLA_COMBINE_HOT_ARGS \
  const int32_t *hot_sched, const int32_t *hot_num_splits, int hot_batch, int hot_R, const float *hot_lacc, const float *hot_oacc

constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt not waited

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// This lane's index, recomputed where it is used (two instructions) rather
// than kept live across a loop whose registers are all taken.
__device__ __forceinline__ int fresh_lane_id() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// A workgroup barrier that lets this wave's last N LDS operations (reads
// issued just before it) stay in flight: LDS operations complete in order, so
// with at most N outstanding every older one (the writes the barrier
// publishes) is done, also when a scalar load is outstanding as well.
template <int N>
__device__ __forceinline__ void lds_barrier_reads_in_flight() {
  static_assert(N > 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest even
  return (unsigned short)(u >> 16);
}

// Asserts to the compiler that a pointer is the same in every lane (it is
// derived from wave-uniform values) so it can live in SGPRs.
__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const unsigned char*)(((unsigned long long)hi << 32) | lo);
}

// Wave-uniform read of read-only metadata through the constant address
// space, so it becomes a scalar load (lgkmcnt) and never waits on vmcnt,
// which counts the page copies in flight.
template <class T>
__device__ __forceinline__ T ld_uniform(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)ptr;
}

// The same read as a vector load (every lane reads the one address; the
// offset register stops the compiler from making it a scalar load), for
// kernels with no copies in flight.  The combine's partial lse values, one
// 64-byte line each, come back faster this way: in an A/B the memory-bound
// step went from 19.7 to 18.8 us.
__device__ __forceinline__ float ld_broadcast(const float* ptr) {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return ptr[z];
}

// ---------------------------------------------------------------------------
// Per-wave page stages.

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
// kStream: nontemporal hint, for data that this launch reads exactly once;
// without it the lines stay in L2 for the other row groups of the part.
template <bool kStream>
__device__ __forceinline__ void issue_stage_slice(const unsigned char* rows, unsigned stage_lds,
                                                  const unsigned dma_off[2], int i) {
  unsigned lane_off = dma_off[i & 1];
  asm volatile("" : "+v"(lane_off));
  const unsigned voff = lane_off + (unsigned)((i >> 1) * 128);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(stage_lds + (unsigned)i * 1024u);
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(rows), "s"(m0)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(rows), "s"(m0)
                 : "memory");
}

template <bool kStream>
__device__ __forceinline__ void issue_stage(const unsigned char* rows, unsigned stage_lds, const unsigned dma_off[2]) {
#pragma unroll
  for (int i = 0; i < kStageSlices; ++i) issue_stage_slice<kStream>(rows, stage_lds, dma_off, i);
}

// Rows past the end of the sequence may hold anything (NaN included): zero
// the V part of this wave's local tokens t >= valid so that P = 0 meets finite V.
__device__ __forceinline__ void zero_stage_tail(LDS_PTR(unsigned char) buf, int valid, int lane) {
  const int t_first = max(valid, 0);
  const int n = (kWaveTokens - t_first) * 8 * 8;      // 16-byte chunks in blocks 0..7
  for (int u = lane; u < n; u += 64) {
    const int t = t_first + (u >> 6), b = (u >> 3) & 7, c = u & 7;
    *(LDS_PTR(u32x4))(buf + b * kStageBlock + t * 128 + c * 16) = u32x4{0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------------------
// Sparse pages ("[DeepSeek-3] FlashMLA", section 11).  Page j of a query
// token's key list is entries 64 j .. 64 j + 63 of its index list; entry e
// names cache row e = page_id * 64 + offset.  A wave holds a page's 64
// entries in one register (lane l: entry l), loaded one page ahead of the
// page's copy by a plain load (the compiler waits for it where it is
// first used, which is after the explicit wait that covers it).  An entry
// is a key if it lies before the list's length and inside the pool; for
// the others the copy reads pool row 0 instead (always in bounds), the row
// is zeroed in LDS and its score masked.
__device__ __forceinline__ int load_page_entries(const Params& p, int req, int j, int lane) {
  const int e = min(kPage * j + lane, p.topk - 1);   // inside the list
  return p.indices[(size_t)req * p.topk + e];
}

struct GatherPage {
  unsigned long long mask;   // bit t: page token t is a key
  // This lane's copy source for slice parity par (local token
  // t = 8 par + lane / 8): cache row rel[par] + t, so that its byte address
  // is kv + rel[par] * 1152 + the lane's dense slice offset.
  int rel[2];
  int row;   // the entry of page token `lane`, pool row 0 if it is not a key (FP8 record gathers)
};

__device__ __forceinline__ GatherPage gather_page(const Params& p, int entry, int j, int L, int tok0, int lane) {
  asm volatile("" : "+v"(entry));   // first use here, after the wait that covers the load
  const bool key = kPage * j + lane < L && (unsigned)entry < (unsigned)p.kv_tokens;
  const int row = key ? entry : 0;
  GatherPage g;
  g.mask = __ballot(key);
  g.row = row;
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int t = 8 * par + (lane >> 3);
    g.rel[par] = __builtin_amdgcn_ds_bpermute((tok0 + t) << 2, row) - t;
  }
  return g;
}

// Copy slice i (block i / 2, tokens 8 (i % 2) .. + 7) of this wave's rows
// of a sparse page: every lane has its own source row.
template <bool kStream>
__device__ __forceinline__ void issue_gather_slice(const Params& p, const GatherPage& g, const unsigned dma_off[2],
                                                   unsigned stage_lds, int i) {
  unsigned lane_off = dma_off[i & 1];
  asm volatile("" : "+v"(lane_off));   // per copy (hoisted, 18 64-bit offsets would not fit in registers)
  const unsigned long long a = (unsigned long long)(size_t)p.kv + (long long)g.rel[i & 1] * kRowBytes +
                               (unsigned)(lane_off + (i >> 1) * 128);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(stage_lds + (unsigned)i * 1024u);
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(a), "s"(m0) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(a), "s"(m0) : "memory");
}

template <bool kStream>
__device__ __forceinline__ void issue_gather(const Params& p, const GatherPage& g, const unsigned dma_off[2],
                                             unsigned stage_lds) {
#pragma unroll
  for (int i = 0; i < kStageSlices; ++i) issue_gather_slice<kStream>(p, g, dma_off, stage_lds, i);
}

// Zero the V part of this wave's slice rows whose bit in `keep` is clear
// (bit t: local token t).
__device__ __forceinline__ void zero_stage_rows(LDS_PTR(unsigned char) buf, unsigned keep, int lane) {
  for (int u = lane; u < kWaveTokens * 64; u += 64) {
    const int t = u >> 6, b = (u >> 3) & 7, c = u & 7;
    if (!((keep >> t) & 1u)) *(LDS_PTR(u32x4))(buf + b * kStageBlock + t * 128 + c * 16) = u32x4{0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------------------
// FP8 cache ("[DeepSeek-3] FlashMLA", section 12): a token's record is 656
// bytes -- the 512 latent dims as e4m3 (OCP), four fp32 scales (scale i for
// dims 128 i .. 128 i + 127), the 64 RoPE dims as bf16.  A wave copies its
// 16 records as they are (10,496 contiguous bytes of LDS) and then
// dequantizes them into its bf16 slice of the page stage: latent value =
// bf16_rne(fp32(e4m3 * scale)), RoPE copied; the rest of the kernel runs on
// bf16 as for a bf16 cache.
constexpr int kFp8Row = 656;
constexpr int kFp8Slice = kWaveTokens * kFp8Row;      // 10,496 bytes: one wave's records
constexpr int kFp8Page = kPage * kFp8Row;             // 41,984 bytes
constexpr int kFp8Copies = (kFp8Slice + 1023) / 1024;   // 11 (the last: 256 bytes, lanes 0..15)
static_assert(kFp8Slice == 10 * 1024 + 256, "FP8 slice copy split");

// Copy i of this wave's records of a block-table page (contiguous).
template <bool kStream>
__device__ __forceinline__ void issue_fp8_copy(const unsigned char* rows, unsigned slice_lds, int i, int lane) {
  unsigned voff = (unsigned)(i * 1024 + lane * 16);
  asm volatile("" : "+v"(voff));
  const unsigned m0 = __builtin_amdgcn_readfirstlane(slice_lds + (unsigned)i * 1024u);
  if (i < kFp8Copies - 1 || lane < 16) {
    if constexpr (kStream)
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(rows), "s"(m0)
                   : "memory");
    else
      asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(rows), "s"(m0)
                   : "memory");
  }
}

// Copy i of this wave's records of a sparse page: chunk u = 64 i + lane of
// the slice is chunk u % 41 of local token u / 41, whose cache row is the
// (clamped) entry held by lane tok0 + u / 41.
template <bool kStream>
__device__ __forceinline__ void issue_fp8_gather(const Params& p, int entry_row, int tok0, unsigned slice_lds, int i,
                                                 int lane) {
  int u = i * 64 + lane;
  asm volatile("" : "+v"(u));   // per copy (hoisted, the 11 copies' offsets would not fit in registers)
  const int t = min((u * 1599) >> 16, kWaveTokens - 1);   // u / 41 for u < 656
  const int row = __builtin_amdgcn_ds_bpermute((tok0 + t) << 2, entry_row);
  const unsigned long long a = (unsigned long long)(size_t)p.kv + (unsigned long long)(unsigned)row * kFp8Row +
                               (unsigned)((u - 41 * t) * 16);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(slice_lds + (unsigned)i * 1024u);
  if (i < kFp8Copies - 1 || lane < 16) {
    if constexpr (kStream)
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(a), "s"(m0) : "memory");
    else
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(a), "s"(m0) : "memory");
  }
}

// Dequantize this wave's 16 records (fp8 slice) into its bf16 stage slice
// (the 16-token layout above).  Block b (dims 64 b .. 64 b + 63) of local
// token t = lane / 8 + 8 r, chunk c = lane % 8 (dims 64 b + 8 c .. + 7): a
// 16-lane pass then reads 8-byte chunks of two records and writes 16-byte
// chunks of two rows, each on distinct LDS banks.  Blocks 0..7 hold the
// e4m3 latent (scale b / 2), block 8 the bf16 RoPE, copied.
//   Every read of the slice is issued before the first write: the compiler
// cannot tell the two stages apart, so a read placed after a write would
// wait for it, and each block would pay a full LDS round trip in turn.
__device__ __forceinline__ void dequant_fp8_slice(LDS_PTR(unsigned char) fp8, LDS_PTR(unsigned char) bf, int lane) {
  const int c = lane & 7;
  u32x2 lat[2][8];
  f32x4 sc[2];
  u32x4 rope[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    LDS_PTR(unsigned char) rec = fp8 + ((lane >> 3) + 8 * r) * kFp8Row;
#pragma unroll
    for (int b = 0; b < 8; ++b) lat[r][b] = *(LDS_PTR(u32x2))(rec + 64 * b + 8 * c);
    sc[r] = *(LDS_PTR(f32x4))(rec + kDv);
    // RoPE dims 512 + 8 c .. + 7 (record bytes 528 + 16 c): block 8, chunk c
    rope[r] = *(LDS_PTR(u32x4))(rec + kDv + 16 + 16 * c);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = (lane >> 3) + 8 * r;
    LDS_PTR(unsigned char) row = bf + t * 128 + ((c ^ stage_swizzle(t)) << 4);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const u32x2 v = lat[r][b];
      const float s = sc[r][b >> 1];
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], false);   // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], true);    // bytes 2, 3
        w[2 * e] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(lo[0] * s), (__bf16)(lo[1] * s)});
        w[2 * e + 1] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(hi[0] * s), (__bf16)(hi[1] * s)});
      }
      *(LDS_PTR(u32x4))(row + b * kStageBlock) = w;
    }
    *(LDS_PTR(u32x4))(row + 8 * kStageBlock) = rope[r];
  }
}

// The FP8 records of a wave's 16 tokens read straight into the K operand
// of S^T = K Q^T in the small kernel's order of the contraction (k-step
// ks, lane (g, c16): token c16, dims 64 (ks / 2) + 16 g + 8 (ks % 2) .. + 7):
// lane (g, c16) holds token c16's latent bytes 64 m + 16 g .. + 15 (k-steps
// 2 m, 2 m + 1), its four tile scales and its RoPE dims 512 + 16 g + 8 i ..
// + 7 (k-step 16 + i).  Sixteen records lie 656 bytes apart, so each
// 16-lane pass reads distinct LDS banks.
struct Fp8Frags {
  u32x4 lat[kDv / 64];
  f32x4 sc;
  u32x4 rope[2];
};

__device__ __forceinline__ Fp8Frags read_fp8_frags(LDS_PTR(unsigned char) slice, int c16, int g) {
  Fp8Frags fr;
  LDS_PTR(unsigned char) rec = slice + c16 * kFp8Row;
#pragma unroll
  for (int m = 0; m < kDv / 64; ++m) fr.lat[m] = *(LDS_PTR(u32x4))(rec + 64 * m + 16 * g);
  fr.sc = *(LDS_PTR(f32x4))(rec + kDv);
#pragma unroll
  for (int i = 0; i < 2; ++i) fr.rope[i] = *(LDS_PTR(u32x4))(rec + kDv + 16 + 32 * g + 16 * i);
  return fr;
}

// K fragment ks in bf16: bf16_rne(fp32(e4m3 * tile scale)) for the latent,
// the stored RoPE; zero for a token that is not a key (keep = 0).
__device__ __forceinline__ u32x4 fp8_k_fragment(const Fp8Frags& fr, int ks, unsigned keep) {
  if (ks >= kDv / 32) return fr.rope[ks - kDv / 32] & keep;
  const u32x4 l = fr.lat[ks >> 1];
  const u32x2 v = (ks & 1) ? u32x2{l[2], l[3]} : u32x2{l[0], l[1]};
  const float s = fr.sc[ks >> 2];
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], false);   // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], true);    // bytes 2, 3
    w[2 * e] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(lo[0] * s), (__bf16)(lo[1] * s)});
    w[2 * e + 1] = __builtin_bit_cast(unsigned, bf16x2{(__bf16)(hi[0] * s), (__bf16)(hi[1] * s)});
  }
  return w & keep;
}

// Q^T fragments (B operand of 16x16x32): query row `row` (masked to zero when
// >= R), dims 32 ks + 8 g .. + 7.
__device__ __forceinline__ void load_q(bf16x8 (&qf)[kQkSteps], const Params& p, int req, int row, int g) {
  const bool ok = row < p.R;
  const unsigned char* qrow = p.q + ((size_t)req * p.R + (ok ? row : 0)) * kRowBytes + g * 16;
  const unsigned keep = ok ? ~0u : 0u;
#pragma unroll
  for (int ks = 0; ks < kQkSteps; ++ks) {
    u32x4 v = *(const u32x4*)(qrow + ks * 64);
    v &= keep;
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Softmax of one 16-row S^T tile against the wave's fixed reference (base 2).
// sv: this lane's 4 scores (tokens 4 g .. + 3 of its row); returns the bf16
// probabilities and adds them (fp32) to l.
__device__ __forceinline__ i16x4 probabilities(f32x4 sv, int g, int valid, float scale_log2, float& m_ref,
                                               float& m_seen, float& l) {
  float x[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    // (softmax_scale >= 0, so masking before or after scaling is the same.)
    x[v] = (4 * g + v) < valid ? sv[v] * scale_log2 : -INFINITY;
    mloc = fmaxf(mloc, x[v]);
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  if (m_ref == -INFINITY) m_ref = mloc;   // the first tile with a visible key sets the reference
  m_seen = fmaxf(m_seen, mloc);
  i16x4 pb;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float pe = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[v] - m_ref);
    l += pe;   // row sum from the fp32 values; only the PV operand is bf16
    pb[v] = __builtin_bit_cast(short, (__bf16)pe);
  }
  return pb;
}

// Merge weights of the four waves' states for one row: M = the largest
// reference among waves with mass, w_i = 2^(m_i - M); returns 1 / sum w_i l_i
// and the row's log2-sum-exp (-inf when the row saw no token).
__device__ __forceinline__ void merge_weights(const float (*st_m)[kRowGroup], const float (*st_l)[kRowGroup], int row,
                                              float (&wgt)[4], float& inv, float& lse2) {
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (st_l[w][row] > 0.f) M = fmaxf(M, st_m[w][row]);
  float lsum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wgt[w] = st_l[w][row] > 0.f ? __builtin_amdgcn_exp2f(st_m[w][row] - M) : 0.f;
    lsum += wgt[w] * st_l[w][row];
  }
  inv = lsum > 0.f ? 1.f / lsum : 0.f;
  lse2 = lsum > 0.f ? M + __builtin_amdgcn_logf(lsum) : -INFINITY;
}

// Writes a finished row: lse (natural log) when the request is not split,
// else the base-2 partial lse of slot `slot`.
// lse is [batch, h_q, s_q]; request `req` is query token req % fold of
// request req / fold (fold = 1 for dense decode).
__device__ __forceinline__ size_t lse_index(const Params& p, int req, int row) {
  const int b = req / p.fold, sv = req - b * p.fold;
  const int s = row / p.h_q, hh = row - s * p.h_q;
  return ((size_t)b * p.h_q + hh) * (size_t)(p.s_q * p.fold) + (size_t)s * p.fold + sv;
}

__device__ __forceinline__ void store_lse(const Params& p, int req, int row, bool split, int slot, float lse2) {
  if (!split) {
    p.lse[lse_index(p, req, row)] = lse2 * kLn2;
  } else {
    p.lacc[(size_t)slot * p.R + row] = lse2;
  }
}

// Four consecutive output columns c .. c + 3 of one row: bf16 to `out` when
// the request is not split, else fp32 to the partial slot.  kNt: the partial
// goes out with the nontemporal hint (the small kernel's choice for large
// partial volumes, see nt_partials; 18-34 % slower for the 128-row kernel's
// 67 MB, so that one keeps plain stores).
template <bool kNt = false>
__device__ __forceinline__ void store_cols4(const Params& p, int req, int row, bool split, int slot, int c, f32x4 v) {
  if (!split) {
    bf16x4 w4;
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = (__bf16)v[e];
    *(bf16x4*)(p.out + ((size_t)req * p.R + row) * kDv + c) = w4;
  } else if constexpr (kNt) {
    __builtin_nontemporal_store(v, (f32x4*)(p.oacc + ((size_t)slot * p.R + row) * kDv + c));
  } else {
    *(f32x4*)(p.oacc + ((size_t)slot * p.R + row) * kDv + c) = v;
  }
}

// A piece of the plan as seen by one part: the request range and, per
// request, its block range, piece index and partial slot.
struct PieceRange {
  int begin_req, end_req, begin_blk, end_blk, begin_piece;
  int first_page;   // block id of page begin_blk of begin_req if the plan carries it, else -1
};

// The whole 32-byte row in one scalar load (one round trip).  Column 6 holds
// the first page's block id + 1 when the caller attached the block table to
// the plan (0 otherwise).
__device__ __forceinline__ PieceRange load_part(const Params& p, int part) {
  const i32x8 v = ld_uniform((const i32x8*)(p.sched + part * MLA_SCHED_INTS));
  return PieceRange{v[0], v[1], v[2], v[3], v[4], v[6] - 1};
}

// What a piece needs of request `req` before its first copies: the length,
// the partial slots [slot0, slot1) and the block ids of pages lo .. lo + 2
// (clamped to the table row: entries past the request's pages are read but
// their values are not used).  The loads do not depend on each other, so
// they cost one round trip together.
struct RequestMeta {
  int L, slot0, slot1, blk[3];
};

// Sparse decode: the length is the count of entries that count (topk, or
// topk_length of the real request, clamped to [0, topk]); no block ids.
__device__ __forceinline__ RequestMeta load_request_sparse(const Params& p, int req) {
  RequestMeta m;
  m.L = p.topk;
  if (p.topk_len) m.L = min(max(ld_uniform(p.topk_len + req / p.fold), 0), p.topk);
  m.slot0 = ld_uniform(p.num_splits + req);
  m.slot1 = ld_uniform(p.num_splits + req + 1);
  m.blk[0] = m.blk[1] = m.blk[2] = 0;
  return m;
}

__device__ __forceinline__ RequestMeta load_request(const Params& p, int req, int lo) {
  const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;
  const int last = p.max_blocks - 1;
  RequestMeta m;
#pragma unroll
  for (int i = 0; i < 3; ++i) m.blk[i] = ld_uniform(bt + min(lo + i, last));
  m.L = ld_uniform(p.seqlens + req);
  m.slot0 = ld_uniform(p.num_splits + req);
  m.slot1 = ld_uniform(p.num_splits + req + 1);
  return m;
}

// ---------------------------------------------------------------------------
// Maps a workgroup id to (part, row group).  Workgroups are dealt to the 8
// XCDs round robin (id % 8), and each XCD takes a contiguous run of
// ceil(parts / 8) parts, all row groups of a part next to each other in its
// dispatch order: the parts of one request (consecutive in the plan) then
// share its query rows, and the row groups of a part its KV pages, through
// that XCD's L2.  The grid is 8 * row_groups * ceil(parts / 8); ids past the
// last part exit.
__device__ __forceinline__ void map_block(const Params& p, int& part, int& rg) {
  // Every kernel argument the prologue needs is made to arrive in one round
  // trip here (the compiler would otherwise load some only after the early
  // exit below, one dependent round trip more before the first page copy).
  asm volatile("" ::"s"(p.sched), "s"(p.seqlens), "s"(p.num_splits), "s"(p.block_table), "s"(p.q), "s"(p.kv),
               "s"(p.out), "s"(p.lse), "s"(p.oacc), "s"(p.lacc));
  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int per = (p.num_parts + 7) / 8;
  rg = slot % p.row_groups;
  part = xcd * per + slot / p.row_groups;
}

// ---------------------------------------------------------------------------
// Small row counts (R = s_q * h_q <= 16), the memory-bound regime: one
// workgroup per part covers every query row.
//   * Each wave copies its 16 token rows of a page into a shared stage (the
//     18 KiB slice layout above); after a barrier every wave sees all four
//     slices of the page.
//   * QK^T is split by tokens: wave w computes S^T (its 16 tokens x 16 rows)
//     with v_mfma_f32_16x16x32_bf16, Q^T in registers, K from its own slice.
//   * Its bf16 probabilities go to LDS as B fragments of the same MFMA shape
//     (32 tokens x 16 rows each, two per page).
//   * PV is split by columns: wave w accumulates O^T for columns
//     128 w .. 128 w + 127 over all 64 tokens of the page (8 tiles of 16x16,
//     32 registers), V^T from transposing reads of all four slices.  Nothing
//     is merged across waves at the end: each wave stores its own columns.
//   * The per-row softmax reference is common to the four waves (the max over
//     the whole first page, exchanged through LDS); row sums are kept per
//     wave and added at the end.
//   * Two barriers per page: the page's slices landed (and every wave is past
//     the previous page: its stage and the P buffer are free), and the P
//     fragments are written.
//   * An FP8 cache: each lane reads its own token's records in the K operand
//     layout and dequantizes them in registers next to the QK^T MFMAs; the
//     latent part also goes to the bf16 stage for PV, which reads it after
//     the P barrier (so the first barrier only frees the stage).
constexpr int kSmallPBytes = 2 * 64 * 16;   // two 32-token P^T fragments
constexpr int kSmallPvLead = 6;             // V^T fragments in flight

// Max / sum over the four 16-lane rows of a wave (lanes c16, c16 + 16,
// c16 + 32, c16 + 48: the four token groups of one query row), with two
// cross-row swaps instead of LDS permutes.
__device__ __forceinline__ float row_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// kSparse: the key lists of sparse decode instead of block-table pages
// (gathered copies, per-token key masks).  kFp8: an FP8 cache; one bf16
// page stage (the dequantized page being computed) and stages of FP8
// records replace the two bf16 stages: two for block-table pages (pages
// j + 1 and j + 2 in flight while page j is computed), one for sparse
// lists (whose entries are loaded by the compiler, whose waits would
// otherwise wait for every copy in flight).
// Row pitch of the small kernel's partial staging: a wave's 128 fp32
// columns (512 bytes) and 16 bytes of padding, which moves each row by four
// banks.
constexpr int kSmallStageRow = 528;
static_assert(4 * kSmallRows * kSmallStageRow <= kPageBytes, "partial staging fits in one page stage");

template <bool kSparse, bool kFp8>
__global__ void __launch_bounds__(256, 1) mla_splitkv_small_kernel(MLA_SPLITKV_HOT_ARGS, Params p_args) {
  const Params p = with_hot_args(p_args, hot_sched, hot_num_parts, hot_row_groups, hot_max_blocks, hot_block_table,
                                 hot_seqlens, hot_num_splits, hot_kv, hot_q);
  constexpr int kF8Stages = kFp8 ? (kSparse ? 1 : 2) : 0;
  // FP8 block-table pages are read one page ahead: page j + 1's records are
  // read into registers (and the next copy issued) while page j's PV runs,
  // then dequantized next to page j + 1's QK^T MFMAs.
  constexpr bool kPipe = kFp8 && !kSparse;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kFp8 ? kPageBytes + kF8Stages * kFp8Page : 2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[kSmallPBytes];
  __shared__ float red[4][kSmallRows];   // per-wave row maxima (FP8: then row sums)
  __shared__ float lsum[4][kSmallRows];  // per-wave row sums of a piece's last page
  __shared__ int vote[4];                // per-wave restart votes

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, rg;
  map_block(p, part, rg);   // rg = 0: one row group
  if (part >= p.num_parts) return;
  const PieceRange pr = load_part(p, part);

  const int g = lane >> 4;     // 16-lane group
  const int c16 = lane & 15;   // MFMA column = query row
  const bool row_ok = c16 < p.R;
  const int tok0 = kWaveTokens * wave;

  LDS_PTR(unsigned char) lds = (LDS_PTR(unsigned char))smem;
  LDS_PTR(unsigned char) pb = (LDS_PTR(unsigned char))pbuf;
  const unsigned wslice = (unsigned)(size_t)lds + wave * kStageBytes;   // this wave's slice of stage 0
  const unsigned dma_off[2] = {stage_dma_offset(lane, 0), stage_dma_offset(lane, 1)};
  // FP8: this wave's records in the FP8 stage (after the bf16 stage).
  LDS_PTR(unsigned char) fp8s = lds + kPageBytes + wave * kFp8Slice;
  const unsigned fslice = (unsigned)(size_t)lds + kPageBytes + wave * kFp8Slice;
  // The request's query rows are staged like a page slice (row r in token
  // slot r) in slice 0 of stage 1 (of the bf16 stage for an FP8 cache);
  // slots >= R copy row 0 instead (in bounds; their fragments are zeroed).
  unsigned q_dma_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int t = 8 * par + (lane >> 3);
    q_dma_off[par] = t < p.R ? dma_off[par] : (unsigned)(((lane & 7) ^ stage_swizzle(t)) << 4);
  }

  // QK A fragment of k-step ks (and the Q^T B fragment, in the same order
  // of the contraction): local token c16, block ks / 2, in-block chunk
  // 2 g + ks % 2, so a lane's two k-steps of a block are 16 adjacent dims.
  int qk_off[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) qk_off[b] = c16 * 128 + (((2 * g + b) ^ stage_swizzle(c16)) << 4);
  // PV A fragment (V^T: 16 columns x 32 tokens of a 32-token step): lane
  // (g, c16) needs column c16 of the tile and step tokens 8 g .. 8 g + 7,
  // from two transposing reads r = 0, 1: the group's 16 lanes read tokens
  // 8 g + 4 r .. + 3 (lane c16: token 8 g + 4 r + c16 / 4, columns
  // 4 (c16 % 4) .. + 3 of the tile) and lane c16 receives column c16.  Step
  // token 8 g + 4 r + c16 / 4 is local token 8 (g % 2) + 4 r + c16 / 4 of
  // slice g / 2 of the step; tile ct of this wave's columns is column block
  // 2 w + ct / 4, in-block chunk 2 (ct % 4) + (c16 % 4) / 2, byte 8 (c16 % 2).
  int pv_off[2][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tl = 8 * (g & 1) + 4 * r + (c16 >> 2);
      pv_off[r][q] = (g >> 1) * kStageBytes + tl * 128 +
                     (((2 * q + ((c16 & 3) >> 1)) ^ stage_swizzle(tl)) << 4) + 8 * (c16 & 1);
    }
  // This lane's 4 probabilities (local tokens 4 g .. + 3 of row c16) are
  // step wave / 2, step tokens 16 (wave % 2) + 4 g .. + 3: B lane
  // (2 (wave % 2) + g / 2, c16), bytes 8 (g % 2) .. + 7.
  const int pw_off = ((wave >> 1) * 64 + (2 * (wave & 1) + (g >> 1)) * 16 + c16) * 16 + 8 * (g & 1);

  // A plan that carries the first page's block id lets the part's first
  // request start its Q and first-page copies right after the plan row,
  // one dependent round trip (the request's metadata) earlier.  The copies
  // go out in the same order as below, so every wait stays as it is.
  const bool early = !kSparse && pr.first_page >= 0 && pr.begin_req <= pr.end_req;   // uniform
  if (early) {
    const unsigned char* qrows = uniform_ptr(p.q + (size_t)pr.begin_req * p.R * kRowBytes);
    const unsigned qslice = (unsigned)(size_t)lds + (kFp8 ? 0 : kPageBytes);
    for (int i = wave; i < kStageSlices; i += 4) issue_stage_slice<false>(qrows, qslice, q_dma_off, i);
    if constexpr (kFp8) {
      const unsigned char* rows = uniform_ptr(p.kv + (size_t)pr.first_page * kFp8Page + (size_t)tok0 * kFp8Row);
#pragma unroll
      for (int i = 0; i < kFp8Copies; ++i) issue_fp8_copy<false>(rows, fslice, i, lane);
    } else {
      issue_stage<false>(uniform_ptr(p.kv + (size_t)pr.first_page * kPageBytes + (size_t)tok0 * kRowBytes), wslice,
                         dma_off);
    }
  }

  for (int req = pr.begin_req; req <= pr.end_req; ++req) {
    const int lo = (req == pr.begin_req) ? pr.begin_blk : 0;
    const bool copied = early && req == pr.begin_req;   // Q and page lo already in flight
    const RequestMeta m = kSparse ? load_request_sparse(p, req) : load_request(p, req, lo);
    // Sparse: the entries of pages lo .. lo + 2, read with the metadata.
    int ent[3] = {0, 0, 0};
    if constexpr (kSparse) {
#pragma unroll
      for (int i = 0; i < 3; ++i) ent[i] = load_page_entries(p, req, lo + i, lane);
    }
    const int L = m.L;
    const int nblk = pages_of(L);
    const int hi = (req == pr.end_req) ? pr.end_blk : nblk;
    const int slot = m.slot0 + ((req == pr.begin_req) ? pr.begin_piece : 0);
    const bool split = m.slot1 - m.slot0 > 1;
    const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;
    auto page_rows = [&](int blk) {
      return uniform_ptr(p.kv + (size_t)blk * kPageBytes + (size_t)tok0 * kRowBytes);
    };
    // FP8: copy this wave's records of a page (block id, or gathered rows) to FP8 stage f.
    auto issue_fp8_page = [&](int blk, int entry_row, int f) {
      const unsigned char* rows = uniform_ptr(p.kv + (size_t)blk * kFp8Page + (size_t)tok0 * kFp8Row);
      const unsigned dst = fslice + (unsigned)(f * kFp8Page);
#pragma unroll
      for (int i = 0; i < kFp8Copies; ++i) {
        if constexpr (kSparse)
          issue_fp8_gather<false>(p, entry_row, tok0, dst, i, lane);
        else
          issue_fp8_copy<false>(rows, dst, i, lane);
      }
    };

    f32x4 o[8];
    float m_ref = -INFINITY, l_run = 0.f;
    float l_tot = 0.f;   // the row's sum over the four waves
    // Q^T fragments (B operand): row c16, dims 32 ks + 8 g .. + 7.  Q is
    // copied once per workgroup, into slice 0 of stage 1, ahead of the first
    // page: wave w copies the 1 KiB pieces w, w + 4, ... of it (a CU moves its
    // bytes at a bounded rate, so four private copies of Q would cost a
    // quarter of a piece's traffic).  Every wave reads it into registers as
    // soon as it has landed, and stage 1 then takes the second page, so
    // both pages are in flight while Q is in use.  (All global reads here
    // are explicit copies with explicit waits: no compiler-tracked load may
    // be outstanding while page copies are in flight.)
    bf16x8 qf[kQkSteps];
    // Sparse: the copy sources and key masks of pages lo and lo + 1 (kept
    // for a restart), computed before any copy is in flight, so that the
    // wait for the entries waits for nothing else.
    GatherPage g0{}, g1{};
    if constexpr (kSparse) {
      g0 = gather_page(p, ent[0], lo, L, tok0, lane);
      g1 = gather_page(p, ent[1], lo + 1, L, tok0, lane);
    }
    if (!copied) {
      const unsigned char* qrows = uniform_ptr(p.q + (size_t)req * p.R * kRowBytes);
      const unsigned qslice = (unsigned)(size_t)lds + (kFp8 ? 0 : kPageBytes);
      for (int i = wave; i < kStageSlices; i += 4) issue_stage_slice<false>(qrows, qslice, q_dma_off, i);
    }
    for (int attempt = 0;; ++attempt) {
      // Sparse: key masks of the current page, of page lo + 1, and of the
      // page whose copy was issued last; the entries of the next page to copy.
      unsigned long long mk_cur = g0.mask, mk_lo1 = g1.mask, mk_pending = 0;
      int ent_next = kFp8 ? ent[1] : ent[2];
      const bool first_in_flight = copied && attempt == 0;
      if constexpr (kFp8) {
        if (lo < hi && !first_in_flight) issue_fp8_page(m.blk[0], g0.row, 0);
        if (kF8Stages == 2 && lo + 1 < hi) issue_fp8_page(m.blk[1], 0, 1);
      } else if constexpr (kSparse) {
        if (lo < hi) issue_gather<false>(p, g0, dma_off, wslice);
      } else {
        if (lo < hi && !first_in_flight) issue_stage<false>(page_rows(m.blk[0]), wslice, dma_off);
      }
      if (attempt == 0) {
        // this wave's pieces of Q (the first pages may still be in flight)
        if (kF8Stages == 2 && lo + 1 < hi)
          wait_vmcnt<2 * kFp8Copies>();
        else if (kFp8 && lo < hi)
          wait_vmcnt<kFp8Copies>();
        else if (!kFp8 && lo < hi)
          wait_vmcnt<kStageSlices>();
        else
          wait_vmcnt<0>();
        lds_barrier();                  // all of Q has landed
        const unsigned keep = row_ok ? ~0u : 0u;
        LDS_PTR(unsigned char) qs = lds + (kFp8 ? 0 : kPageBytes);
#pragma unroll
        for (int ks = 0; ks < kQkSteps; ++ks) {
          u32x4 v = *(LDS_PTR(u32x4))(qs + (ks >> 1) * kStageBlock + qk_off[ks & 1]);
          v &= keep;
          qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
        lds_barrier();                  // every wave has read Q: stage 1 is free again
      }
      if (lo + 1 < hi && !kFp8) {
        if constexpr (kSparse)
          issue_gather<false>(p, g1, dma_off, wslice + kPageBytes);
        else
          issue_stage<false>(page_rows(m.blk[1]), wslice + kPageBytes, dma_off);
      }
      int next_blk = kF8Stages == 1 ? m.blk[1] : m.blk[2];   // block ids are read one page ahead of their copy

#pragma unroll
      for (int ct = 0; ct < 8; ++ct) o[ct] = f32x4{0, 0, 0, 0};
      float m_seen = -INFINITY;
      l_run = 0.f;
      bool restart = false;

      // FP8 block-table pages: the records of the page being computed, in
      // the K operand layout (page lo's read here, the others during the
      // previous page's PV).
      Fp8Frags frn;
      if constexpr (kPipe) {
        if (lo < hi) {
          if (lo + 1 < hi)
            wait_vmcnt<kFp8Copies>();   // page lo + 1's records may still be in flight
          else
            wait_vmcnt<0>();
          frn = read_fp8_frags(fp8s, c16, g);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // FP8 stage 0 has been read
          if (lo + 2 < hi) {
            issue_fp8_page(next_blk, 0, 0);
            next_blk = ld_uniform(bt + min(lo + 3, p.max_blocks - 1));
          }
        }
      }

      for (int j = lo; j < hi; ++j) {
        const int stage = kFp8 ? 0 : (j - lo) & 1;
        LDS_PTR(unsigned char) buf = lds + stage * kPageBytes;
        // This wave's slice of page j (the next page's copy, if any, is issued
        // below, after the barrier).
        if constexpr (kPipe) {
          // (page j's records were waited for and dequantized during page j - 1)
        } else if (j == lo && lo + 1 < hi && !kFp8) {
          wait_vmcnt<kStageSlices>();
        } else {
          wait_vmcnt<0>();
        }
        LDS_PTR(unsigned char) own = buf + wave * kStageBytes;
        u32x4 kf[kQkSteps];
        if constexpr (kPipe) {
          if (j > lo) lds_barrier();   // every wave is done with page j - 1: the bf16 stage and P buffer are free
        } else if constexpr (kFp8) {
          // Sparse lists (one FP8 stage): its records are in; once every wave
          // is done with page j - 1 (the bf16 stage and the P buffer are free)
          // each lane reads its token's records in the K operand layout, and
          // the FP8 stage takes the records of page j + 1.  The K fragments
          // are dequantized in registers and written to the bf16 stage for PV
          // (latent only; PV reads it after the barrier that publishes P).
          if (j > lo) lds_barrier();
          const Fp8Frags fr = read_fp8_frags(fp8s, c16, g);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // its reads of the FP8 stage are done
          if (j + 1 < hi) {
            const GatherPage gn = gather_page(p, ent_next, j + 1, L, tok0, lane);
            issue_fp8_page(0, gn.row, 0);
            mk_pending = gn.mask;
            ent_next = load_page_entries(p, req, j + 2, lane);
          }
          const unsigned keep = ((mk_cur >> (tok0 + c16)) & 1ull) != 0 ? ~0u : 0u;
#pragma unroll
          for (int ks = 0; ks < kQkSteps; ++ks) {
            kf[ks] = fp8_k_fragment(fr, ks, keep);
            if (ks < kDv / 32) *(LDS_PTR(u32x4))(own + (ks >> 1) * kStageBlock + qk_off[ks & 1]) = kf[ks];
          }
        }
        if constexpr (!kFp8) {
          if constexpr (kSparse) {
            const unsigned keep = (unsigned)(mk_cur >> tok0) & 0xFFFFu;
            if (keep != 0xFFFFu) zero_stage_rows(own, keep, lane);
          } else {
            const int valid = min(kPage, L - j * kPage);
            if (valid - tok0 < kWaveTokens) zero_stage_tail(own, valid - tok0, lane);
          }
          lds_barrier();   // page j is visible; every wave is past page j - 1
          // Page j + 1 goes to the stage page j - 1 held (pages lo, lo + 1 were
          // issued ahead of the loop).  (A third page in flight from the start,
          // held in registers, was measured slower: every page then lands late.)
          if (j > lo && j + 1 < hi) {
            if constexpr (kSparse) {
              const GatherPage gn = gather_page(p, ent_next, j + 1, L, tok0, lane);
              issue_gather<false>(p, gn, dma_off, wslice + ((j + 1 - lo) & 1) * kPageBytes);
              mk_pending = gn.mask;
              ent_next = load_page_entries(p, req, j + 2, lane);
            } else {
              issue_stage<false>(page_rows(next_blk), wslice + ((j + 1 - lo) & 1) * kPageBytes, dma_off);
              next_blk = ld_uniform(bt + min(j + 2, p.max_blocks - 1));
            }
          }
#pragma unroll
          for (int ks = 0; ks < kQkSteps; ++ks)
            kf[ks] = *(LDS_PTR(u32x4))(own + (ks >> 1) * kStageBlock + qk_off[ks & 1]);
        }

        // ---- S^T (this wave's 16 tokens x 16 rows) = K Q^T, three chains.
        f32x4 sacc[3] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
        if constexpr (kPipe) {
          // FP8 block-table pages: K fragment ks is dequantized right before
          // its MFMA (in the shadow of the previous ones) and its latent part
          // written to the bf16 stage for PV.
          auto qk = [&](unsigned keep) {
#pragma unroll
            for (int ks = 0; ks < kQkSteps; ++ks) {
              const u32x4 k = fp8_k_fragment(frn, ks, keep);
              if (ks < kDv / 32) *(LDS_PTR(u32x4))(own + (ks >> 1) * kStageBlock + qk_off[ks & 1]) = k;
              sacc[ks % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k), qf[ks],
                                                                      sacc[ks % 3], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          };
          // (uniform: a page whose 16 tokens of this wave are all keys needs no mask)
          if (L - j * kPage - tok0 >= kWaveTokens)
            qk(~0u);
          else
            qk(tok0 + c16 < L - j * kPage ? ~0u : 0u);
        } else {
#pragma unroll
          for (int ks = 0; ks < kQkSteps; ++ks)
            sacc[ks % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks],
                                                                    sacc[ks % 3], 0, 0, 0);
        }
        const f32x4 sv = sacc[0] + sacc[1] + sacc[2];

        // ---- softmax against the common reference (base 2).
        const int vis = row_keys(p, L, c16) - j * kPage;   // keys of this page row c16 sees (may be <= 0 or > 64)
        const unsigned kw = (unsigned)(mk_cur >> tok0) & 0xFFFFu;   // sparse: keys among this wave's tokens
        float x[4], mloc = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // (softmax_scale >= 0, so masking before or after scaling is the same.)
          const bool key = kSparse ? ((kw >> (4 * g + v)) & 1u) != 0 : tok0 + 4 * g + v < vis;
          x[v] = key ? sv[v] * p.scale_log2 : -INFINITY;
          mloc = fmaxf(mloc, x[v]);
        }
        mloc = row_max4(mloc);   // this wave's tokens of row c16
        // A row's reference is the whole page's row max of the first page in
        // which it sees a key, the same in every wave (exchanged through LDS).
        // m_ref is equal across waves, so the vote is uniform.
        if (__any(m_ref == -INFINITY)) {
          if (g == 0) red[wave][c16] = mloc;
          lds_barrier();
          if (m_ref == -INFINITY) m_ref = fmaxf(fmaxf(red[0][c16], red[1][c16]), fmaxf(red[2][c16], red[3][c16]));
        }
        m_seen = fmaxf(m_seen, mloc);
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;   // no key seen yet: every x is -inf
        i16x4 pk;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float pe = __builtin_amdgcn_exp2f(x[v] - m_use);   // masked tokens: exp2(-inf) = 0
          l_run += pe;   // row sum from the fp32 values; only the PV operand is bf16
          pk[v] = __builtin_bit_cast(short, (__bf16)pe);
        }
        *(LDS_PTR(i16x4))(pb + pw_off) = pk;
        // bf16 pages: the last page's row sums travel with its probabilities,
        // so the epilogue needs no exchange of its own (0.3 us of the
        // memory-bound step in an A/B; with FP8 records 0.1 us slower, so
        // that kernel keeps the exchange in its epilogue).
        if (!kFp8 && j == hi - 1) {
          const float lw = row_sum4(l_run);
          if (g == 0) lsum[wave][c16] = lw;
        }
        // A row max more than 2^64 above the reference: every wave redoes the
        // piece with the exact maxima (first attempt only, so at most twice).
        if (attempt == 0) {
          const bool any_bad = __any(mloc > m_ref + kRefHeadroom);
          if (lane == 0) vote[wave] = any_bad;
        }
        lds_barrier();   // every wave's probabilities (and vote) are in LDS
        if (attempt == 0) restart |= (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
        if (!kFp8 && j == hi - 1) l_tot = (lsum[0][c16] + lsum[1][c16]) + (lsum[2][c16] + lsum[3][c16]);

        // ---- O^T (this wave's 128 columns x 16 rows) += V^T P^T, two steps of
        // 32 tokens, 8 column tiles each.
        // Software pipelined: V^T fragment i + kSmallPvLead is read right after
        // the MFMA of fragment i (i = 8 step + ct).
        {
          auto vread = [&](int i) {
            LDS_PTR(unsigned char) a = buf + (i >> 3) * 2 * kStageBytes + (2 * wave + ((i & 7) >> 2)) * kStageBlock;
            const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_off[0][i & 3]));
            const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_off[1][i & 3]));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
          };
          // FP8 block-table pages: page j + 1's records (landed; page j + 2's
          // copies may still be in flight) are read with the first V^T
          // fragments, and its FP8 stage takes page j + 3 after the MFMAs.
          const bool next = kPipe && j + 1 < hi;
          if constexpr (kPipe) {
            if (next) {
              if (j + 2 < hi)
                wait_vmcnt<kFp8Copies>();
              else
                wait_vmcnt<0>();
              frn = read_fp8_frags(fp8s + ((j + 1 - lo) & 1) * kFp8Page, c16, g);
            }
          }
          const bf16x8 pB0 = *(LDS_PTR(bf16x8))(pb + lane * 16);
          const bf16x8 pB1 = *(LDS_PTR(bf16x8))(pb + (64 + lane) * 16);
          bf16x8 vf[kSmallPvLead];
#pragma unroll
          for (int i = 0; i < kSmallPvLead; ++i) vf[i] = vread(i);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            o[i & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[i % kSmallPvLead], i < 8 ? pB0 : pB1, o[i & 7], 0, 0, 0);
            if (i + kSmallPvLead < 16) vf[i % kSmallPvLead] = vread(i + kSmallPvLead);
            __builtin_amdgcn_sched_barrier(0);
          }
          if constexpr (kPipe) {
            if (next) {
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this FP8 stage has been read
              if (j + 3 < hi) {
                issue_fp8_page(next_blk, 0, (j + 1 - lo) & 1);
                next_blk = ld_uniform(bt + min(j + 4, p.max_blocks - 1));
              }
            }
          }
        }
        if constexpr (kSparse) mk_cur = j == lo && !kFp8 ? mk_lo1 : mk_pending;
      }
      wait_vmcnt<0>();
      if (!restart) break;
      // Restart: the exact row maxima over all four waves become the reference.
      lds_barrier();   // every wave is past the last page
      if (g == 0) red[wave][c16] = m_seen;
      lds_barrier();
      m_ref = fmaxf(fmaxf(red[0][c16], red[1][c16]), fmaxf(red[2][c16], red[3][c16]));
      lds_barrier();   // red is read before it is written again
    }

    // ---- epilogue: row sums over the four waves (bf16 pages: already known);
    // each wave stores its columns.
    if constexpr (kFp8) {
      const float lw = row_sum4(l_run);
      lds_barrier();   // every wave is done with red
      if (g == 0) red[wave][c16] = lw;
      lds_barrier();
      l_tot = (red[0][c16] + red[1][c16]) + (red[2][c16] + red[3][c16]);
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    // In the O^T accumulator lane (g, c16) holds row c16, columns 4 g .. + 3 of the tile.
    if (!kFp8 && split) {
      // The partial goes out in whole 128-byte lines: this wave's 16 rows x
      // 128 columns pass through a free stage (rows 528 bytes apart, so a
      // write's 16 rows fall on distinct banks) and each store covers two
      // rows.  Stored straight from the accumulator layout, a store writes
      // 64-byte halves of 16 lines, which the nontemporal path does not merge
      // (10.4 MB written for 7.2 MB of partials on the memory-bound
      // workload); staged, the step went from 19.2 to 18.3 us in an A/B with
      // bitwise the same output.  (FP8 records: 18.1 against 18.3 us the
      // other way round, so that kernel keeps the direct stores.)
      // (in the stage that does not hold the last page: other waves may
      // still be reading that one)
      LDS_PTR(unsigned char) stg =
          lds + (((hi - 1 - lo) & 1) ? 0 : kPageBytes) + wave * (kSmallRows * kSmallStageRow);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        *(LDS_PTR(f32x4))(stg + c16 * kSmallStageRow + (16 * ct + 4 * g) * 4) = o[ct] * inv;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's staging writes are done (its own region)
#pragma unroll
      for (int i = 0; i < kSmallRows / 2; ++i) {
        const int rr = 2 * i + (lane >> 5), ch = lane & 31;
        const f32x4 v = *(LDS_PTR(f32x4))(stg + rr * kSmallStageRow + ch * 16);
        f32x4* dst = (f32x4*)(p.oacc + ((size_t)slot * p.R + rr) * kDv + 128 * wave + 4 * ch);
        if (rr < p.R) {
          if (p.nt_partials)
            __builtin_nontemporal_store(v, dst);
          else
            *dst = v;
        }
      }
    } else if (row_ok) {
      if (p.nt_partials) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) store_cols4<true>(p, req, c16, split, slot, 128 * wave + 16 * ct + 4 * g, o[ct] * inv);
      } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) store_cols4<false>(p, req, c16, split, slot, 128 * wave + 16 * ct + 4 * g, o[ct] * inv);
      }
    }
    if (wave == 0 && g == 0 && row_ok) store_lse(p, req, c16, split, slot, lse2);
    lds_barrier();   // red is read; the next piece may reuse LDS
  }
}

// ---------------------------------------------------------------------------
// Larger row counts (R > 16): one workgroup per (part, group of 32 query
// rows); the R / 32 workgroups of a part are placed on one XCD, next to each
// other in dispatch order, so every KV page they all stream comes from HBM
// once and from that XCD's L2 for the others.
//   * S^T is computed per 16-row half with v_mfma_f32_16x16x32_bf16; each K
//     fragment read from LDS feeds both halves.
//   * The two halves' bf16 probabilities are rearranged with one
//     v_permlane16_swap per dword into the B operand of
//     v_mfma_f32_32x32x16_bf16 (8 consecutive tokens of one row per lane), so
//     O^T (512 x 32 rows) += V^T (512 x 16 tokens) P^T runs at the full
//     matrix rate: 16 MFMAs per page, V^T from two transposing reads each.
//   * The 32-row x 512 fp32 accumulator is 256 registers per wave; each wave
//     has its own (its tokens' share), merged through LDS in two rounds of
//     256 columns at the end of a piece.

constexpr int kParkCols = 8;   // 32-column tiles parked per merge round (32 KiB per wave)
constexpr int kQkLead = 6;     // K fragment reads in flight ahead of the QK MFMAs
constexpr int kPvLead = 4;     // V^T fragments (two reads each) in flight ahead of the PV MFMAs
static_assert(kQkSteps == kStageSlices && kDv / 32 == 16, "copy slices: 9 in QK^T, 8 + 1 in PV");

__global__ void __launch_bounds__(256, 1) mla_splitkv_kernel(MLA_SPLITKV_HOT_ARGS, Params p_args) {
  const Params p = with_hot_args(p_args, hot_sched, hot_num_parts, hot_row_groups, hot_max_blocks, hot_block_table,
                                 hot_seqlens, hot_num_splits, hot_kv, hot_q);
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * 2 * kStageBytes];
  __shared__ float st_m[4][kRowGroup], st_l[4][kRowGroup];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, rg;
  map_block(p, part, rg);
  if (part >= p.num_parts) return;
  const PieceRange pr = load_part(p, part);

  const int g = lane >> 4;     // 16-lane group
  const int c16 = lane & 15;   // 16x16 MFMA column = query row within a half
  const int row0 = rg * kRowGroup;
  const int tok0 = kWaveTokens * wave;

  LDS_PTR(unsigned char) wlds = (LDS_PTR(unsigned char))smem + wave * 2 * kStageBytes;
  const unsigned wlds0 = (unsigned)(size_t)wlds;
  const unsigned dma_off[2] = {stage_dma_offset(lane, 0), stage_dma_offset(lane, 1)};

  // QK A fragment of k-step ks: local token c16, logical chunk 4 ks + g.
  int qk_off[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) qk_off[b] = c16 * 128 + (((4 * b + g) ^ stage_swizzle(c16)) << 4);
  // PV A fragment (32x32x16) of column tile ct, read r: the 16-lane group g
  // covers columns 32 ct + 16 (g % 2) .. + 15 and tokens 8 (g / 2) + 4 r .. + 3;
  // lane c16 reads token 8 (g / 2) + 4 r + c16 / 4 at columns 32 ct + 16 (g % 2)
  // + 4 (c16 % 4) .. + 3 and receives column 32 ct + 16 (g % 2) + c16 of the
  // group's 4 tokens.  Column block ct / 2, in-block chunk
  // 4 (ct % 2) + 2 (g % 2) + (c16 % 4) / 2, byte 8 (c16 % 2).
  int pv_off[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int t = 8 * (g >> 1) + 4 * r + (c16 >> 2);
      pv_off[r][par] = t * 128 + (((4 * par + 2 * (g & 1) + ((c16 & 3) >> 1)) ^ stage_swizzle(t)) << 4) + 8 * (c16 & 1);
    }

  for (int req = pr.begin_req; req <= pr.end_req; ++req) {
    const int lo = (req == pr.begin_req) ? pr.begin_blk : 0;
    const RequestMeta m = load_request(p, req, lo);
    const int L = m.L;
    const int nblk = pages_of(L);
    const int hi = (req == pr.end_req) ? pr.end_blk : nblk;
    const int slot = m.slot0 + ((req == pr.begin_req) ? pr.begin_piece : 0);
    const bool split = m.slot1 - m.slot0 > 1;
    const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;
    auto page_rows = [&](int blk) {
      return uniform_ptr(p.kv + (size_t)blk * kPageBytes + (size_t)tok0 * kRowBytes);
    };

    f32x16 o[kDv / 32];
    float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    for (int attempt = 0;; ++attempt) {
      if (lo < hi) issue_stage<false>(page_rows(m.blk[0]), wlds0, dma_off);
      bf16x8 qf[2][kQkSteps];
      load_q(qf[0], p, req, row0 + c16, g);
      load_q(qf[1], p, req, row0 + 16 + c16, g);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

#pragma unroll
      for (int ct = 0; ct < kDv / 32; ++ct) o[ct] = f32x16{};
      float m_seen[2] = {-INFINITY, -INFINITY};
      l_run[0] = l_run[1] = 0.f;

      // Block-table entries are read one page ahead of their use.
      int next_blk = ld_uniform(bt + (lo + 1 < hi ? lo + 1 : lo));
      for (int j = lo; j < hi; ++j) {
        const int stage = (j - lo) & 1;
        LDS_PTR(unsigned char) buf = wlds + stage * kStageBytes;
        // The next page's 18 copy slices go to the other stage (which held
        // page j - 1, whose reads completed in the previous iteration), one
        // after each QK^T step, so that the copy issue overlaps the MFMAs
        // instead of stalling the wave in one burst.  On the last
        // page the current page is copied again instead (harmless: that
        // stage is not read again in this piece), which keeps the loop body
        // free of branches.
        const unsigned char* nrows =
            uniform_ptr(p.kv + (size_t)next_blk * kPageBytes + (size_t)tok0 * kRowBytes);
        next_blk = ld_uniform(bt + (j + 2 < hi ? j + 2 : j));
        const unsigned nlds = wlds0 + (stage ^ 1) * kStageBytes;
        wait_vmcnt<0>();                 // page j (copied during the previous iteration)
        const int valid = min(kPage, L - j * kPage) - tok0;   // valid local tokens (may be <= 0)
        if (valid < kWaveTokens) zero_stage_tail(buf, valid, lane);

        // ---- S^T (16 tokens x 32 rows) = K Q^T: each K fragment feeds both
        // 16-row halves.  Software pipelined: the read of fragment ks + kQkLead
        // is issued right after the MFMAs of fragment ks (the scheduling fences
        // keep that order), so kQkLead reads are always in flight.
        f32x4 sacc[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
        {
          auto kread = [&](int ks) {
            return __builtin_bit_cast(bf16x8, *(LDS_PTR(u32x4))(buf + (ks >> 1) * kStageBlock + qk_off[ks & 1]));
          };
          bf16x8 kf[kQkLead];
#pragma unroll
          for (int i = 0; i < kQkLead; ++i) kf[i] = kread(i);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < kQkSteps; ++ks) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
              sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % kQkLead], qf[t][ks], sacc[t], 0, 0, 0);
            if (ks + kQkLead < kQkSteps) kf[ks % kQkLead] = kread(ks + kQkLead);
            issue_stage_slice<false>(nrows, nlds, dma_off, ks);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // The first PV fragments do not depend on P: their reads overlap the softmax.
        auto vread = [&](int ct) {
          LDS_PTR(unsigned char) a = buf + (ct >> 1) * kStageBlock;
          const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_off[0][ct & 1]));
          const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv_off[1][ct & 1]));
          return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vf[kPvLead];
#pragma unroll
        for (int i = 0; i < kPvLead; ++i) vf[i] = vread(i);
        i16x4 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          pb[t] = probabilities(sacc[t], g, row_keys(p, L, row0 + 16 * t + c16) - j * kPage - tok0, p.scale_log2,
                                m_ref[t], m_seen[t], l_run[t]);

        // ---- P^T as the 32x32x16 B operand: lane 32 h + n needs tokens
        // 8 h .. 8 h + 7 of row n.  Half t = n / 16 holds them in lanes
        // 32 h + n % 16 (tokens 8 h .. + 3) and 32 h + 16 + n % 16 (+ 4 .. + 7);
        // swapping 16-lane rows between the two halves' registers delivers both.
        const u32x2 h0 = __builtin_bit_cast(u32x2, pb[0]), h1 = __builtin_bit_cast(u32x2, pb[1]);
        const auto s0 = __builtin_amdgcn_permlane16_swap(h0[0], h1[0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(h0[1], h1[1], false, false);
        const bf16x8 pB = __builtin_bit_cast(bf16x8, u32x4{s0[0], s1[0], s0[1], s1[1]});

        // ---- O^T (512 x 32 rows) += V^T (512 x 16 tokens) P^T, software
        // pipelined like QK^T: kPvLead V^T fragments (two transposing reads
        // each) stay in flight ahead of the MFMAs.
        {
#pragma unroll
          for (int ct = 0; ct < kDv / 32; ++ct) {
            o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ct % kPvLead], pB, o[ct], 0, 0, 0);
            if (ct + kPvLead < kDv / 32) vf[ct % kPvLead] = vread(ct + kPvLead);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      wait_vmcnt<0>();   // the last copy, before a restart or the merge reuses the stages
      // One retry with the exact maxima always suffices: every probability is then <= 1.
      if (attempt > 0 || !__any(m_seen[0] > m_ref[0] + kRefHeadroom || m_seen[1] > m_ref[1] + kRefHeadroom)) break;
      m_ref[0] = m_seen[0];
      m_ref[1] = m_seen[1];
    }

    // ---- merge the four waves' states.  Row sums first: lane (g, c16) holds
    // 4 tokens of rows c16 and 16 + c16.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float lw = l_run[t] + __shfl_xor(l_run[t], 16);
      lw += __shfl_xor(lw, 32);
      if (g == 0) {
        st_m[wave][16 * t + c16] = m_ref[t];
        st_l[wave][16 * t + c16] = lw;
      }
    }
    // In the O^T accumulator lane l holds row n = l % 32 and, in element
    // 4 i + e, column 32 ct + 8 i + 4 (l / 32) + e.
    // (From a lane index read here, so that the compiler does not compute
    // the epilogue's store addresses ahead of the piece loop and keep them
    // in scratch: the page loop leaves no registers free.)
    const int le = fresh_lane_id();
    const int n = le & 31;
    const int row = row0 + n;
    float wgt[4], inv = 0.f, lse2 = 0.f;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      // Park this wave's column tiles 8 round .. + 7 in its own stages (its
      // copies are complete), then every wave finalises two of them.
#pragma unroll
      for (int k = 0; k < kParkCols; ++k) {
        const f32x16 v = o[kParkCols * round + k];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(LDS_PTR(f32x4))(wlds + ((k * 4 + q4) * 64 + lane) * 16) =
              f32x4{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
      }
      lds_barrier();
      if (round == 0) merge_weights(st_m, st_l, n, wgt, inv, lse2);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int k = 2 * wave + k2;
        const int ct = kParkCols * round + k;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int w = 0; w < 4; ++w)
            acc += wgt[w] * *(LDS_PTR(f32x4))((LDS_PTR(unsigned char))smem + w * 2 * kStageBytes +
                                              ((k * 4 + q4) * 64 + lane) * 16);
          if (row < p.R) store_cols4(p, req, row, split, slot, 32 * ct + 8 * q4 + 4 * (le >> 5), acc * inv);
        }
      }
      lds_barrier();   // the parked tiles are read; the stages may be reused
    }
    if (wave == 0 && le < 32 && row < p.R) {
      Params pe = p;   // h_q through an opaque copy: its division constant is not kept from the kernel start
      asm volatile("s_mov_b32 %0, %1" : "=s"(pe.h_q) : "s"(p.h_q));
      store_lse(pe, req, row, split, slot, lse2);
    }
  }
}

// ---------------------------------------------------------------------------
// Wide row groups (R >= 128): one workgroup per (part, group of 128 query
// rows), so each KV page enters a CU once per 128 rows instead of once per
// 32 (the per-CU path from L2 is the narrower resource for the 32-row kernel)
// and two LDS stages cover two full page times of copy latency.
//   * Each wave still copies its own 16 token rows of a page (the 18 KiB
//     slice layout above), but both stages are shared: a barrier after the
//     copies land makes every slice visible to every wave.
//   * QK^T is split by rows: wave w computes S^T (64 tokens x 32 rows
//     32 w .. 32 w + 31) with v_mfma_f32_32x32x16_bf16, Q in registers, K
//     fragments from the four slices.  Each wave owns the softmax state of its
//     32 rows (so no cross-wave merge is needed at the end).
//   * Its bf16 probabilities go to LDS straight from the S^T accumulator as
//     PV B fragments (the token order inside a 16-token step is the
//     accumulator's; the V^T reads use the same order).
//   * PV is split by columns: wave w accumulates O^T for columns
//     128 w .. 128 w + 127 of all 128 rows (4 x 4 tiles of 32x32, 256
//     registers); every V^T fragment feeds four MFMAs.
//   * Two barriers per page: after the P fragments are written, and after PV
//     (P buffer and the page's stage free; the next page's slices landed).
constexpr int kWideTiles = kWideRows / 32;                 // 32-row tiles per group (= waves)
constexpr int kPFragBytes = kWideTiles * 4 * 64 * 16;      // P^T: 4 row tiles x 4 token steps x 64 lanes x 16 B
constexpr int kQkSteps16 = kDqk / 16;                      // 36 k-steps of the 32x32x16 MFMA
constexpr int kWideQkLead = 4;                             // K fragment reads in flight
constexpr int kWideSoftmaxPieces = 22;                     // pieces of one tile's softmax

// Softmax state of one 32-token S^T tile.  Lane l holds row l % 32 and, in
// element 4 i + e, token 8 i + 4 (l / 32) + e of the tile.  The pieces (each
// rides in the shadow of one MFMA; no piece depends on a result of the same
// piece):
//   0, 1   max of this lane's 16 scores (partial maxima, then their max)
//   2      row max over both lane halves, scaled
//   3      the first tile sets the reference; running max, restart test
//   4 .. 21   the 16 elements through a three-stage pipeline: exponent
//          argument of element k - 4, exp2 of element k - 5, row sum (and
//          bf16 pack of each completed pair) of element k - 6; each completed
//          8-token half goes to LDS as a PV B fragment.
// A 32x32x16 MFMA leaves about 16 clk of the wave's issue time in its
// shadow (measured: three VALU operations and one v_exp_f32 between two
// MFMAs keep the matrix core's rate; a whole element pair's stages, seven
// VALU operations and two v_exp_f32, stall it), so a piece is at most one
// element's stages.  Every stage's inputs and results pass through empty
// volatile asm statements so that the compiler keeps each piece in its gap
// (left to itself it merged stages across the copy branches, which put up
// to 17 VALU operations and 4 exp2 between two MFMAs and none elsewhere).
// Piece k of a window of n MFMAs rides after MFMA wide_piece_step(k, n).
constexpr int wide_piece_step(int k, int nsteps) { return 1 + k * (nsteps - 2) / (kWideSoftmaxPieces - 1); }
// Inverse as a table (piece riding after MFMA step i, or -1), indexed by the
// unrolled step so that it folds to a constant.
struct WidePieceMap {
  signed char at[kDqk / 16];
};
constexpr WidePieceMap wide_piece_map(int nsteps) {
  WidePieceMap m{};
  for (int i = 0; i < kDqk / 16; ++i) m.at[i] = -1;
  for (int k = 0; k < kWideSoftmaxPieces; ++k) m.at[wide_piece_step(k, nsteps)] = (signed char)k;
  return m;
}
constexpr WidePieceMap kWidePiecesQk = wide_piece_map(kDqk / 16);   // tile 0 along QK^T of tile 1 (36 MFMAs)
constexpr WidePieceMap kWidePiecesPv = wide_piece_map(32);          // tile 1 along PV of tokens 0 .. 31 (32 MFMAs)
static_assert(wide_piece_step(kWideSoftmaxPieces - 1, kDqk / 16) == kDqk / 16 - 1, "pieces fit the QK^T window");
static_assert(wide_piece_step(kWideSoftmaxPieces - 1, 32) == 31, "pieces fit the PV window");
struct WideSoftmax {
  float mp[6], mloc;
  float ex[16];
  u32x4 pk[2];
};

// O^T += V^T P^T on the matrix cores with the accumulator pinned to AGPRs
// (volatile, like the QK^T MFMAs: their order against the softmax pieces'
// pins is the program's):
// O (256 registers per lane) stays in the accumulation registers for the
// whole piece, which leaves the architectural VGPRs to Q, the S^T tiles and
// the softmax.  The compiler does not see inside the statement, so the code
// around it keeps the hazard distances itself: operands come from LDS reads
// (waited for by the compiler's counters) and reads of the accumulator are
// preceded by wide_acc_settle().  The operands are passed as 32-bit words:
// as bf16 vectors the compiler sometimes rebuilt a fragment with v_perm or
// v_bfi right before the statement, and an MFMA that reads a VGPR a VALU op
// has just written needs two wait states that nothing here would insert
// (the compiler's hazard checks do not look inside the statement; a build
// with a fifth K fragment in flight read stale operands that way).
__device__ __forceinline__ void pv_mfma(f32x16& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// S^T tiles in architectural VGPRs (so they never compete with O for the
// accumulation registers); the first step of a tile starts from zero.  Its
// result is an early-clobber output: a 16-register MFMA result must not
// overlap the instruction's own A or B operand (the compiler's definitions
// of these MFMAs carry the same constraint).
__device__ __forceinline__ void qk_mfma(f32x16& acc, const u32x4& a, const u32x4& b, bool first) {
  if (first)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// Wait states between the last matrix op writing the accumulators and any
// other access to them (a 16-pass MFMA result needs 18).
__device__ __forceinline__ void wide_acc_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// kSparse: the key lists of sparse decode instead of block-table pages
// (gathered copies, per-token key masks).  kFp8: an FP8 cache; one bf16
// page stage (the dequantized page being computed) and one stage of FP8
// records (the next page, in flight) replace the two bf16 stages.
template <bool kStream, bool kSparse, bool kFp8>
__global__ void __launch_bounds__(256, 1) mla_splitkv_wide_kernel(MLA_SPLITKV_HOT_ARGS, Params p_args) {
  const Params p = with_hot_args(p_args, hot_sched, hot_num_parts, hot_row_groups, hot_max_blocks, hot_block_table,
                                 hot_seqlens, hot_num_splits, hot_kv, hot_q);
  // Two page stages (4 slices of 18 KiB each) and the P^T exchange buffer: 160 KiB
  // (FP8: a bf16 stage and an FP8 stage, 129 KiB).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kFp8 ? kPageBytes + kFp8Page : 2 * kPageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char pbuf[kPFragBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int part, rg;
  map_block(p, part, rg);
  if (part >= p.num_parts) return;
  const PieceRange pr = load_part(p, part);

  const int h = lane >> 5;     // which half of the 32x32 MFMA k slots
  const int n = lane & 31;     // 32x32 MFMA column = query row within a tile
  const int row0 = rg * kWideRows;
  const int r = row0 + 32 * wave + n;   // the row this lane owns in QK^T / softmax
  const bool row_ok = r < p.R;
  const int tok0 = kWaveTokens * wave;

  LDS_PTR(unsigned char) lds = (LDS_PTR(unsigned char))smem;
  LDS_PTR(unsigned char) pb = (LDS_PTR(unsigned char))pbuf;
  const unsigned lds0 = (unsigned)(size_t)lds;
  const unsigned dma_off[2] = {stage_dma_offset(lane, 0), stage_dma_offset(lane, 1)};
  // FP8: this wave's records in the FP8 stage (after the bf16 stage).
  LDS_PTR(unsigned char) fp8s = lds + kPageBytes + wave * kFp8Slice;
  const unsigned fslice = lds0 + kPageBytes + wave * kFp8Slice;

  // QK A fragment (32x32x16) of token tile tt, k-step ks: token m = 32 tt + n
  // = slice 2 tt + n / 16, local row n % 16; dims 16 ks + 8 h .. + 7 =
  // block ks / 4, in-block chunk 2 (ks % 4) + h.
  int kq[4];   // tile 0; tile 1 is 2 slices further
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = n & 15;
    kq[q] = (n >> 4) * kStageBytes + t * 128 + (((2 * q + h) ^ stage_swizzle(t)) << 4);
  }
  // PV A fragment (V^T, 32 columns x 16 tokens of slice kk) in the token order
  // of the S^T accumulator: lane (group G, index Lq) reads token
  // 4 (G / 2) + Lq / 4 (read 0) or that + 8 (read 1) at columns
  // 32 ct + 16 (G % 2) + 4 (Lq % 4) .. + 3.
  const int G = lane >> 4, Lq = lane & 15;
  int pv[2][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int t = 4 * (G >> 1) + (Lq >> 2) + 8 * rd;
      pv[rd][par] = t * 128 + (((4 * par + 2 * (G & 1) + ((Lq & 3) >> 1)) ^ stage_swizzle(t)) << 4) + 8 * (Lq & 1);
    }

  for (int req = pr.begin_req; req <= pr.end_req; ++req) {
    const int lo = (req == pr.begin_req) ? pr.begin_blk : 0;
    const RequestMeta m = kSparse ? load_request_sparse(p, req) : load_request(p, req, lo);
    const int L = m.L;
    const int nblk = pages_of(L);
    const int hi = (req == pr.end_req) ? pr.end_blk : nblk;
    const int slot = m.slot0 + ((req == pr.begin_req) ? pr.begin_piece : 0);
    const bool split = m.slot1 - m.slot0 > 1;
    const int32_t* bt = p.block_table + (size_t)req * p.max_blocks;
    auto page_rows = [&](int blk) {
      return uniform_ptr(p.kv + (size_t)blk * kPageBytes + (size_t)tok0 * kRowBytes);
    };
    // FP8: copy this wave's records of a page (block id, or gathered rows).
    auto issue_fp8_page = [&](int blk, int entry_row) {
      const unsigned char* rows = uniform_ptr(p.kv + (size_t)blk * kFp8Page + (size_t)tok0 * kFp8Row);
#pragma unroll
      for (int i = 0; i < kFp8Copies; ++i) {
        if constexpr (kSparse)
          issue_fp8_gather<kStream>(p, entry_row, tok0, fslice, i, lane);
        else
          issue_fp8_copy<kStream>(rows, fslice, i, lane);
      }
    };
    f32x16 o[kWideTiles][4];   // O^T tiles: row tile x this wave's 4 column tiles
    float m_ref = -INFINITY, l_run = 0.f;
    for (int attempt = 0;; ++attempt) {
      // Sparse: the entries of pages lo and lo + 1 (read with the metadata on
      // the first attempt, again on a restart rather than kept live).
      int ent_next = 0;
      GatherPage g0{};
      if constexpr (kSparse) {
        const int ent0 = load_page_entries(p, req, lo, lane);
        ent_next = load_page_entries(p, req, lo + 1, lane);
        g0 = gather_page(p, ent0, lo, L, tok0, lane);
      }
      // The first page's copies.  Sparse lists go out ahead of Q; with a block
      // table Q's loads (mostly L2 hits) go first and the page copies right
      // behind them, so Q has landed when the page does (the loads complete in
      // order): steps 0.5-1 % shorter on the 4K-token and long-context workloads.
      auto issue_first_page = [&]() {
        if (lo < hi) {
          if constexpr (kFp8)
            issue_fp8_page(m.blk[0], g0.row);
          else if constexpr (kSparse)
            issue_gather<kStream>(p, g0, dma_off, lds0 + wave * kStageBytes);
          else
            issue_stage<kStream>(page_rows(m.blk[0]), lds0 + wave * kStageBytes, dma_off);
        }
      };
      if constexpr (kSparse) issue_first_page();
      // Q^T fragments (B operand): row r, dims 16 ks + 8 h .. + 7.
      u32x4 qf[kQkSteps16];
      unsigned keep;
      {
        // (the row address from a lane index read here: kept from the kernel
        // start, it would be spilled with the page loop's registers in use)
        const int lq = fresh_lane_id(), rq = row0 + 32 * wave + (lq & 31);
        const bool okq = rq < p.R;
        const unsigned char* qrow = p.q + ((size_t)req * p.R + (okq ? rq : 0)) * kRowBytes + (lq >> 5) * 16;
        keep = okq ? ~0u : 0u;
#pragma unroll
        for (int ks = 0; ks < kQkSteps16; ++ks) qf[ks] = *(const u32x4*)(qrow + ks * 32);
      }
      if constexpr (!kSparse) issue_first_page();
      // Q and the first page (a wait the compiler sees, so it inserts none
      // inside the page loop, whose waits cover only the copies it issues).
      // Rows past R take zero queries, masked once Q is in.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
      for (int ks = 0; ks < kQkSteps16; ++ks) qf[ks] &= keep;
#pragma unroll
      for (int a = 0; a < kWideTiles; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[a][c] = f32x16{};
      float m_seen = -INFINITY;
      l_run = 0.f;
      float l_part[4] = {0.f, 0.f, 0.f, 0.f};
      bool bad = false;          // a row max outgrew this lane's reference
      int next_blk = m.blk[1];   // copied only if lo + 1 < hi
      unsigned long long mk_cur = g0.mask;   // sparse: key mask of page j

      for (int j = lo; j < hi; ++j) {
        const int stage = kFp8 ? 0 : (j - lo) & 1;
        LDS_PTR(unsigned char) buf = lds + stage * kPageBytes;
        // Page j: this wave's slice has landed; zero its rows past the end of
        // the sequence, then the barrier makes all four slices visible (and
        // every wave is past the previous page's PV: P buffer and the other
        // stage are free).
        wait_vmcnt<0>();
        if constexpr (kFp8) {
          // Its records are in; once every wave is done with page j - 1 the
          // bf16 stage takes page j, dequantized.
          if (j > lo) lds_barrier();
          dequant_fp8_slice(fp8s, buf + wave * kStageBytes, lane);
        }
        if constexpr (kSparse) {
          const unsigned keep = (unsigned)(mk_cur >> tok0) & 0xFFFFu;
          if (keep != 0xFFFFu) zero_stage_rows(buf + wave * kStageBytes, keep, fresh_lane_id());
        } else {
          const int valid = min(kPage, L - j * kPage);
          if (__builtin_expect(valid < kPage, 0)) zero_stage_tail(buf + wave * kStageBytes, valid - tok0, fresh_lane_id());
        }
        lds_barrier();
        // The next page's 18 slices go to the other stage during QK^T (none
        // on the last page: re-copying the current page instead, branch-free,
        // cost 5-8 % more HBM reads on short pieces).
        const bool has_next = j + 1 < hi;   // uniform
        const unsigned char* nrows =
            uniform_ptr(p.kv + (size_t)next_blk * kPageBytes + (size_t)tok0 * kRowBytes);
        const unsigned nlds = lds0 + (stage ^ 1) * kPageBytes + wave * kStageBytes;
        unsigned long long mk_next = 0;
        GatherPage gn{};
        const unsigned char* f8rows = nullptr;   // FP8 block-table pages: the next page's records
        // The next page's copies go out during QK^T of tile 0 (every two
        // MFMAs for bf16 rows, every three for the 11 copies of FP8
        // records, into the FP8 stage this wave dequantized from, whose
        // reads the barrier above has ordered); dense bf16 pages spread
        // theirs over both tiles.
        if constexpr (kSparse) {
          gn = gather_page(p, ent_next, j + 1, L, tok0, lane);   // each lane keeps its row offsets
          mk_next = gn.mask;
          ent_next = load_page_entries(p, req, j + 2, lane);   // covered by the next page's wait
        } else {
          if constexpr (kFp8) f8rows = uniform_ptr(p.kv + (size_t)next_blk * kFp8Page + (size_t)tok0 * kFp8Row);
          next_blk = ld_uniform(bt + (j + 2 < hi ? j + 2 : j));
        }

        // ---- S^T (64 tokens x this wave's 32 rows) in two 32-token tiles.
        // The softmax of each tile rides along the next MFMA stream (tile 0
        // with QK^T of tile 1, tile 1 with PV of tokens 0 .. 31), so its VALU
        // work and exp2 latency hide under the matrix cores.
        WideSoftmax sm[2];
        // Element v of a tile is a key this lane's row sees iff its offset is
        // below lim; a tile is ragged (masking needed) for this workgroup if
        // it is for the row that sees the fewest keys.
        const int lim = row_keys(p, L, r) - j * kPage - 4 * h;
        const int vis_min = (p.causal ? L - (p.s_q - 1) : L) - j * kPage;
        // One piece of tile tt's softmax (see WideSoftmax); k is a constant
        // after unrolling.  The scores are read from the accumulator as they
        // are needed; tokens past the end of the sequence (last page only)
        // are masked in both passes.
        auto softmax_piece = [&](int tt, int k, f32x16& sacc) {
          WideSoftmax& t = sm[tt];
          const bool ragged = kSparse ? (unsigned)(mk_cur >> (32 * tt)) != 0xFFFFFFFFu   // uniform
                                      : vis_min < 32 * tt + 32;
          // Element v of the tile is a real token.  Only evaluated inside the
          // ragged branches: `lim_in` is re-materialised there so that the
          // compares cannot be hoisted onto the full-tile path.
          auto ok = [&](int v, int lim_in) {
            if constexpr (kSparse)
              return ((unsigned)lim_in >> (8 * (v >> 2) + (v & 3))) & 1u;
            else
              return 32 * tt + 8 * (v >> 2) + (v & 3) < lim_in;
          };
          auto branch_lim = [&]() {
            int l2;
            if constexpr (kSparse)
              // this lane's 16 tokens of the tile: bits 8 (v / 4) + v % 4 (the
              // tile's 32-bit word is uniform; only the lane half's shift is not)
              asm volatile("v_mov_b32 %0, %1 ; ragged tile" : "=v"(l2) : "v"((unsigned)(mk_cur >> (32 * tt)) >> (4 * (fresh_lane_id() >> 5))));
            else
              asm volatile("v_mov_b32 %0, %1 ; ragged tile" : "=v"(l2) : "v"(lim));
            return l2;
          };
          // Pins (empty volatile asm): a value passed through one is computed
          // before it and read after it, which holds each stage in its gap.
          auto pinf = [](float& x) { asm volatile("" : "+v"(x)); };
          auto pins = [&](int v) {
            float x = sacc[v];
            asm volatile("" : "+v"(x));
            sacc[v] = x;
          };
          if (k == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) pins(v);
            // Partial maxima (five independent max3s).
            if (__builtin_expect(ragged, 0)) {
              // A real branch (the statement cannot be speculated): full
              // tiles must not pay for the masking selects.  Masked scores
              // become -inf in place; the exponent arguments below are
              // clamped with max(., -inf), which turns the NaN of
              // -inf * 0 (softmax_scale = 0) or -inf + inf (a row with no
              // key seen yet) into -inf, so exp2 gives 0 there.
              const int l2 = branch_lim();
#pragma unroll
              for (int v = 0; v < 16; ++v) sacc[v] = ok(v, l2) ? sacc[v] : -INFINITY;
#pragma unroll
              for (int i = 0; i < 5; ++i) t.mp[i] = fmaxf(fmaxf(sacc[3 * i], sacc[3 * i + 1]), sacc[3 * i + 2]);
              t.mp[5] = sacc[15];
            } else {
#pragma unroll
              for (int i = 0; i < 5; ++i) t.mp[i] = fmaxf(fmaxf(sacc[3 * i], sacc[3 * i + 1]), sacc[3 * i + 2]);
              t.mp[5] = sacc[15];
            }
#pragma unroll
            for (int i = 0; i < 6; ++i) pinf(t.mp[i]);
          } else if (k == 1) {
            t.mloc = fmaxf(fmaxf(fmaxf(t.mp[0], t.mp[1]), t.mp[2]), fmaxf(fmaxf(t.mp[3], t.mp[4]), t.mp[5]));
            pinf(t.mloc);
          } else if (k == 2) {
            // The other half of the row's tokens sits in lane l ^ 32
            // (softmax_scale >= 0: the max commutes with the scaling).
            // A tile with no key has max -inf, and -inf * 0 (softmax_scale = 0)
            // is NaN: the clamp keeps it -inf, so such a tile sets no reference.
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t.mloc), __float_as_uint(t.mloc), false, false);
            t.mloc = fmaxf(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * p.scale_log2, -INFINITY);
            pinf(t.mloc);
          } else if (k == 3) {
            if (m_ref == -INFINITY) m_ref = t.mloc;   // the first tile in which the row sees a key
            m_seen = fmaxf(m_seen, t.mloc);
            bad |= t.mloc > m_ref + kRefHeadroom;
            pinf(m_ref);
            pinf(m_seen);
          } else {
            // Three-stage pipeline over the 16 elements, so that no stage
            // waits on a result of the same piece: exponent argument of
            // element k - 4, exp2 of element k - 5, row sum (and bf16 pack of
            // a completed pair) of element k - 6.
            const int ea = k - 4, ee = k - 5, es = k - 6;
            if (es >= 0 && es < 16) {
              l_part[es & 3] += t.ex[es];   // four independent partial row sums
              asm volatile("" : "+v"(l_part[es & 3]));
              if (es & 1) {
                unsigned w = __builtin_bit_cast(unsigned, bf16x2{(__bf16)t.ex[es - 1], (__bf16)t.ex[es]});
                asm volatile("" : "+v"(w));
                t.pk[es >> 3][(es >> 1) & 3] = w;
              }
              if (es == 7 || es == 15) {   // an 8-token half is complete: to LDS as a PV B fragment
                const int half = es >> 3;
                *(LDS_PTR(u32x4))(pb + ((wave * 4 + 2 * tt + half) * 64 + lane) * 16) = t.pk[half];
              }
            }
            if (ee >= 0 && ee < 16) {
              t.ex[ee] = __builtin_amdgcn_exp2f(t.ex[ee]);
              pinf(t.ex[ee]);
            }
            if (ea >= 0 && ea < 16) {
              pins(ea);
              t.ex[ea] = fmaxf(__builtin_fmaf(sacc[ea], p.scale_log2, -m_ref), -INFINITY);
              pinf(t.ex[ea]);
            }
          }
        };

        f32x16 sacc[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          auto kread = [&](int ks) {
            return *(LDS_PTR(u32x4))(buf + 2 * tt * kStageBytes + (ks >> 2) * kStageBlock + kq[ks & 3]);
          };
          u32x4 kf[kWideQkLead];
#pragma unroll
          for (int i = 0; i < kWideQkLead; ++i) kf[i] = kread(i);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < kQkSteps16; ++ks) {
            qk_mfma(sacc[tt], kf[ks % kWideQkLead], qf[ks], ks == 0);
            if (ks + kWideQkLead < kQkSteps16) kf[ks % kWideQkLead] = kread(ks + kWideQkLead);
            if constexpr (!kSparse && !kFp8)
              if (ks % 4 == 0 && has_next) issue_stage_slice<kStream>(nrows, nlds, dma_off, 9 * tt + ks / 4);
            if constexpr (kSparse && !kFp8)
              if (tt == 0 && ks % 2 == 0 && has_next) issue_gather_slice<kStream>(p, gn, dma_off, nlds, ks / 2);
            if constexpr (kFp8)
              if (tt == 0 && ks % 3 == 0 && ks / 3 < kFp8Copies && has_next) {
                if constexpr (kSparse)
                  issue_fp8_gather<kStream>(p, gn.row, tok0, fslice, ks / 3, lane);
                else
                  issue_fp8_copy<kStream>(f8rows, fslice, ks / 3, lane);
              }
            // Tile 0's softmax, one piece after each of 22 of these MFMAs.
            if (tt == 1 && ks == 1) wide_acc_settle();
            if (tt == 1 && kWidePiecesQk.at[ks] >= 0) softmax_piece(0, kWidePiecesQk.at[ks], sacc[0]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- O^T (this wave's 128 columns x 128 rows) += V^T P^T, one
        // 16-token step kk at a time; tile 1's softmax runs along kk = 0, 1.
        // Accumulator o[a][c] holds row tile (wave + a) % 4, so that a = 0 is
        // the wave's own rows, whose P^T fragments it still holds in registers
        // (the bytes it wrote to LDS): the four V^T fragments of a step are
        // read before the barrier that publishes the probabilities (the page's
        // V was visible since the page barrier), and the first four MFMAs after
        // it need no LDS read, while the other row tiles' P^T fragments arrive.
        // Within a step: row tile a, then column tile c; each V^T fragment of
        // the next step is read once its last use in this step is issued, each
        // P^T fragment likewise; the softmax pieces (if any) sit between single
        // MFMAs.
        auto vread = [&](int cl, int kk) {
          const int ct = 4 * wave + cl;
          LDS_PTR(unsigned char) a = buf + kk * kStageBytes + (ct >> 1) * kStageBlock;
          const u32x2 a0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv[0][ct & 1])));
          const u32x2 a1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(i16x4))(a + pv[1][ct & 1])));
          return u32x4{a0[0], a0[1], a1[0], a1[1]};
        };
        u32x4 vf[4];
        auto pv_block = [&](int kk0, bool with_softmax) {
          u32x4 pf[kWideTiles];   // pf[a], a >= 1: row tile (wave + a) % 4 from LDS
          auto pread = [&](int i, int a) {
            pf[a] = *(LDS_PTR(u32x4))(pb + ((((wave + a) & 3) * 4 + kk0 + i) * 64 + lane) * 16);
          };
#pragma unroll
          for (int a = 1; a < kWideTiles; ++a) pread(0, a);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int a = 0; a < kWideTiles; ++a) {
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int m = 16 * i + 4 * a + c;
                pv_mfma(o[a][c], vf[c], a == 0 ? sm[kk0 >> 1].pk[i] : pf[a]);
                if (i == 0 && a == kWideTiles - 1) vf[c] = vread(c, kk0 + 1);
                if (i == 0 && a > 0 && c == 3) pread(1, a);
                if (with_softmax && kWidePiecesPv.at[m] >= 0) softmax_piece(1, kWidePiecesPv.at[m], sacc[1]);
                __builtin_amdgcn_sched_barrier(0);
              }
            }
          }
        };
#pragma unroll
        for (int c = 0; c < 4; ++c) vf[c] = vread(c, 0);
        lds_barrier_reads_in_flight<8>();   // every wave's tile-0 probabilities are in LDS
        wide_acc_settle();   // tile 1's scores are read next
        pv_block(0, true);
#pragma unroll
        for (int c = 0; c < 4; ++c) vf[c] = vread(c, 2);
        lds_barrier_reads_in_flight<8>();   // every wave's tile-1 probabilities are in LDS
        pv_block(2, false);
        if constexpr (kSparse) mk_cur = mk_next;
      }
      wait_vmcnt<0>();   // no copy is outstanding (kept for the restart path's refill)
      wide_acc_settle();
      l_run = (l_part[0] + l_part[1]) + (l_part[2] + l_part[3]);
      // If a row max outgrew its reference by more than 2^64 in any wave,
      // every wave redoes the piece with the largest maxima seen as references
      // (once; exact maxima bound every probability by 1).  The attempt has
      // run to its end (its results are discarded), which keeps a single exit
      // from the page loop; the vote is taken once per piece, through LDS.
      // Only the first attempt may ask for a restart (whatever the data, even
      // NaN, the piece is processed at most twice).
      if (attempt != 0) break;
      {
        const bool wave_bad = __any(bad);
        lds_barrier();   // every wave is done with the P buffer
        if (lane == 0) *(LDS_PTR(int))(pb + 4 * wave) = wave_bad ? 1 : 0;
        lds_barrier();
        const int votes = *(LDS_PTR(int))(pb) | *(LDS_PTR(int))(pb + 4) | *(LDS_PTR(int))(pb + 8) | *(LDS_PTR(int))(pb + 12);
        if (votes == 0) break;   // (uniform; the epilogue's first barrier orders these reads before its writes)
      }
      lds_barrier();     // every wave is past the last page before the stages are refilled
      m_ref = m_seen;
    }

    // ---- epilogue: each wave owns rows 32 w + n for l and lse; publish 1 / l
    // so that every wave can normalise its columns of all 128 rows.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse2 = l_tot > 0.f ? m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    // (The LDS and store addresses are derived from a lane index read here,
    // so that the compiler does not compute them once ahead of the piece loop
    // and keep them in scratch: the page loop leaves no registers free.)
    const int le = fresh_lane_id(), ne = le & 31, he = le >> 5;
    lds_barrier();   // every wave is done with the P buffer
    if (he == 0) *(LDS_PTR(float))(pb + (wave * 32 + ne) * 4) = inv;
    lds_barrier();
    Params pe = p;   // R and h_q through opaque copies: nothing derived from them is kept from the kernel start
    asm volatile("s_mov_b32 %0, %1" : "=s"(pe.h_q) : "s"(p.h_q));
    asm volatile("s_mov_b32 %0, %1" : "=s"(pe.R) : "s"(p.R));
    // (accumulator o[a] holds row tile (wave + a) % 4)
    float inv_rows[kWideTiles];
#pragma unroll
    for (int a = 0; a < kWideTiles; ++a) inv_rows[a] = *(LDS_PTR(float))(pb + (((wave + a) & 3) * 32 + ne) * 4);
#pragma unroll
    for (int a = 0; a < kWideTiles; ++a) {
      const int ra = row0 + 32 * ((wave + a) & 3) + ne;
      if (ra >= pe.R) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int ct = 4 * wave + c;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_cols4(pe, req, ra, split, slot, 32 * ct + 8 * i + 4 * he,
                      f32x4{o[a][c][4 * i], o[a][c][4 * i + 1], o[a][c][4 * i + 2], o[a][c][4 * i + 3]} *
                          inv_rows[a]);
      }
    }
    const int re = row0 + 32 * wave + ne;
    if (he == 0 && re < pe.R) store_lse(pe, req, re, split, slot, lse2);
    lds_barrier();   // the 1 / l table is read; the next piece may reuse the buffers
  }
}

// ---------------------------------------------------------------------------
// Merge the partial (O_i, lse_i) of every split request (the log-sum-exp
// merge of the attention-kernel page and the overview page, section 7):
// M = max lse_i, w_i = 2^(lse_i - M), out = sum w_i O_i / sum w_i,
// lse = M + log2(sum w_i) (then converted to natural log).  Rows of requests
// that are not split are skipped (the main kernel wrote them).
//   Each lane owns columns 4 l .. 4 l + 3 and 256 + 4 l .. + 3, so each of
// a split's two loads reads 1 KB in one piece (0.44 us of the memory-bound
// step against 8 consecutive columns a lane), and issues the loads of a
// chunk of splits at once, so a wave pays one memory round trip per chunk.
// The chunk is the smallest of 2, 4 and kCombineChunk that holds all of the
// wave's splits (the last chunk's missing entries repeat the last split with
// weight 0, so a smaller chunk issues fewer such loads: 0.4 us of the
// memory-bound step, 14 splits a pair over 4 waves).  If no request has more
// than kCombineChunk pieces (the schedule table says), each wave merges one
// (request, row) pair on its own (many short merges: no LDS, no barrier);
// otherwise a workgroup merges one pair, wave w taking splits w, w + 4, ...,
// and the four states meet in LDS (few long merges).
constexpr int kCombineWaves = 4;
constexpr int kCombineChunk = 8;

// Online merge of splits first, first + step, ... (count of them) of one
// pair into (M, l, a0, a1), kChunk splits a round trip.
template <int kChunk>
__device__ __forceinline__ void combine_chunks(const float* lrow, const float* orow, size_t lstride, size_t ostride,
                                               int first, int step, int count, float& M, float& l, f32x4& a0,
                                               f32x4& a1) {
  for (int k0 = 0; k0 < count; k0 += kChunk) {
    float li[kChunk];
    f32x4 b0[kChunk], b1[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int i = first + step * min(k0 + u, count - 1);   // clamped: duplicates get weight 0 below
      li[u] = ld_broadcast(lrow + (size_t)i * lstride);
      b0[u] = *(const f32x4*)(orow + (size_t)i * ostride);
      b1[u] = *(const f32x4*)(orow + (size_t)i * ostride + kDv / 2);
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (k0 + u < count) Mc = fmaxf(Mc, li[u]);
    if (Mc == -INFINITY) continue;   // nothing with mass so far (uniform)
    const float sa = __builtin_amdgcn_exp2f(M - Mc);   // M = -inf gives 0
    a0 *= sa;
    a1 *= sa;
    l *= sa;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float w = (k0 + u < count) ? __builtin_amdgcn_exp2f(li[u] - Mc) : 0.f;   // lse = -inf gives 0
      a0 += w * b0[u];
      a1 += w * b1[u];
      l += w;
    }
    M = Mc;
  }
}

// combine_chunks with the chunk picked by the split count (uniform over the wave).
__device__ __forceinline__ void combine_splits(const float* lrow, const float* orow, size_t lstride, size_t ostride,
                                               int first, int step, int count, float& M, float& l, f32x4& a0,
                                               f32x4& a1) {
  if (count <= 2)
    combine_chunks<2>(lrow, orow, lstride, ostride, first, step, count, M, l, a0, a1);
  else if (count <= 4)
    combine_chunks<4>(lrow, orow, lstride, ostride, first, step, count, M, l, a0, a1);
  else
    combine_chunks<kCombineChunk>(lrow, orow, lstride, ostride, first, step, count, M, l, a0, a1);
}

__device__ __forceinline__ void combine_store(const Params& p, int req, int row, int lane, float M, float l, f32x4 a0,
                                              f32x4 a1) {
  const float inv = l > 0.f ? 1.f / l : 0.f;
  unsigned short* o = p.out + ((size_t)req * p.R + row) * kDv + lane * 4;
  u32x2 w0, w1;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    w0[e] = (unsigned)f32_to_bf16(a0[2 * e] * inv) | ((unsigned)f32_to_bf16(a0[2 * e + 1] * inv) << 16);
    w1[e] = (unsigned)f32_to_bf16(a1[2 * e] * inv) | ((unsigned)f32_to_bf16(a1[2 * e + 1] * inv) << 16);
  }
  *(u32x2*)o = w0;
  *(u32x2*)(o + kDv / 2) = w1;
  if (lane == 0) p.lse[lse_index(p, req, row)] = l > 0.f ? (M + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

__global__ void __launch_bounds__(kCombineWaves * 64) mla_combine_kernel(MLA_COMBINE_HOT_ARGS, Params p_args) {
  Params p = p_args;
  p.sched = hot_sched;
  p.num_splits = hot_num_splits;
  p.batch = hot_batch;
  p.R = hot_R;
  p.lacc = const_cast<float*>(hot_lacc);
  p.oacc = const_cast<float*>(hot_oacc);
  __shared__ f32x4 red_o[kCombineWaves][2][64];
  __shared__ float red_m[kCombineWaves], red_l[kCombineWaves];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pairs = p.batch * p.R;
  const size_t ostride = (size_t)p.R * kDv;
  // The piece counts of both layouts' first pairs are read together with
  // the table's largest piece count (one round trip), and the next pair's
  // while the current one is merged.
  auto splits_of = [&](int pair, int& slot0, int& slot1) {
    const int req = min(pair, pairs - 1) / p.R;
    slot0 = ld_uniform(p.num_splits + req);
    slot1 = ld_uniform(p.num_splits + req + 1);
  };
  const int first_w = blockIdx.x * kCombineWaves + wave, first_g = blockIdx.x;
  int sw0, sw1, sg0, sg1;
  splits_of(first_w, sw0, sw1);
  splits_of(first_g, sg0, sg1);
  const int max_pieces = ld_uniform(p.sched + 5);   // the schedule table's largest piece count
  if (max_pieces <= 1) return;
  if (max_pieces <= kCombineChunk) {
    // Many short merges: one pair per wave.
    for (int pair = first_w; pair < pairs; pair += gridDim.x * kCombineWaves) {
      const int req = pair / p.R, row = pair - req * p.R;
      const int slot0 = sw0;
      const int n = sw1 - sw0;
      splits_of(pair + gridDim.x * kCombineWaves, sw0, sw1);
      if (n <= 1) continue;   // uniform over the wave
      float M = -INFINITY, l = 0.f;
      f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
      combine_splits(p.lacc + (size_t)slot0 * p.R + row, p.oacc + ((size_t)slot0 * p.R + row) * kDv + lane * 4, p.R,
                     ostride, 0, 1, n, M, l, a0, a1);
      combine_store(p, req, row, lane, M, l, a0, a1);
    }
    return;
  }
  // Few long merges: one pair per workgroup, wave w taking splits w, w + 4, ...
  for (int pair = first_g; pair < pairs; pair += gridDim.x) {
    const int req = pair / p.R, row = pair - req * p.R;
    const int slot0 = sg0;
    const int n = sg1 - sg0;
    splits_of(pair + gridDim.x, sg0, sg1);
    if (n <= 1) continue;   // uniform over the workgroup
    const int nw = (n - wave + kCombineWaves - 1) / kCombineWaves;   // this wave's splits
    float M = -INFINITY, l = 0.f;
    f32x4 a0 = {0, 0, 0, 0}, a1 = {0, 0, 0, 0};
    combine_splits(p.lacc + (size_t)slot0 * p.R + row, p.oacc + ((size_t)slot0 * p.R + row) * kDv + lane * 4, p.R,
                   ostride, wave, kCombineWaves, nw, M, l, a0, a1);
    red_o[wave][0][lane] = a0;
    red_o[wave][1][lane] = a1;
    if (lane == 0) {
      red_m[wave] = M;
      red_l[wave] = l;
    }
    __syncthreads();
    if (wave == 0) {
      float Mt = -INFINITY;
#pragma unroll
      for (int w = 0; w < kCombineWaves; ++w) Mt = fmaxf(Mt, red_m[w]);
      float lt = 0.f;
      f32x4 t0 = {0, 0, 0, 0}, t1 = {0, 0, 0, 0};
      if (Mt != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kCombineWaves; ++w) {
          const float sw = __builtin_amdgcn_exp2f(red_m[w] - Mt);   // an empty wave (-inf) gives 0
          t0 += sw * red_o[w][0][lane];
          t1 += sw * red_o[w][1][lane];
          lt += sw * red_l[w];
        }
      }
      combine_store(p, req, row, lane, Mt, lt, t0, t1);
    }
    __syncthreads();   // red_* are reused by the next pair
  }
}

// ---------------------------------------------------------------------------
// The split planner on the GPU ("FlashMLA new-kernel deep dive", Tile
// Scheduler: the pages run their planner as a one-warp kernel), so that a
// captured decode step can replan from lengths that change on the device.
// It produces the host planner's table (planner.cpp: same payload rule, same
// greedy walk, same evening of single-request runs), then empty rows
// (begin_req = 1 > end_req = 0, which every split-KV kernel skips) up to
// num_parts, column 5 = the largest piece count in every row, and the
// per-request prefix of pieces.
//   The walk is not stepped part by part.  One wave holds 64 requests at a
// time; a ballot over the in-chunk prefix of costs (n_b + F) places the whole
// run of requests that fit in the capacity left, and a request that does not
// fit is settled in O(1): its first piece takes what the part has left beyond
// F (or the part closes if that is nothing), every fresh part after it is
// filled with payload - F of its blocks, k = (rem - 1) / (payload - F) times,
// and its last piece opens the part the walk continues in.  Each fresh part
// records where it begins (request, block, piece index, and the block count
// of that request) in LDS; a part ends where the next one begins, so the rows
// are then written one lane per part, by all kPlanWaves waves (the walk
// itself is one wave's).
constexpr int kPlanMaxBatch = 1 << 16;
constexpr int kPlanMaxParts = 4096;
constexpr int kPlanWaves = 4;

__device__ __forceinline__ long long readlane64(long long v, int lane) {
  const int lo = __builtin_amdgcn_readlane((int)(v & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), lane);
  return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__global__ void __launch_bounds__(kPlanWaves * 64) mla_plan_kernel(const int32_t* seqlens, int batch, int num_parts,
                                                                 int F, int32_t* sched, int32_t* num_splits,
                                                                 const int32_t* block_table, int max_blocks,
                                                                 int num_blocks) {
  __shared__ int pb_req[kPlanMaxParts], pb_blk[kPlanMaxParts], pb_piece[kPlanMaxParts];
  __shared__ int pb_n[kPlanMaxParts];   // blocks of the request each part begins in
  __shared__ int walk_out[2];   // parts the walk used, largest piece count
  auto blocks_of = [](int L) { return pages_of(L); };   // negative lengths count as 0
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // total = sum (n_b + F); payload = ceil(total / parts) + F
    long long part_sum = 0;
    for (int b = lane; b < batch; b += 64) part_sum += blocks_of(seqlens[b]) + F;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part_sum += __shfl_xor(part_sum, off);
    const long long total = readlane64(part_sum, 0);
    const long long P = (total + num_parts - 1) / num_parts + F;
    const long long D = P - F;    // blocks a piece may take in a part of its own
    const int last = num_parts - 1;

    int p = 0;                    // the part the walk is in
    long long cap = P;            // capacity left in part p
    int acc = 0, max_pieces = 1;  // pieces of the requests before this chunk; largest piece count
    if (lane == 0) {
      pb_req[0] = pb_blk[0] = pb_piece[0] = 0;
      pb_n[0] = blocks_of(seqlens[0]);
      num_splits[0] = 0;
    }
    for (int base = 0; base < batch; base += 64) {
      const int cnt = min(64, batch - base);
      const int n = lane < cnt ? blocks_of(seqlens[base + lane]) : 0;
      long long z = (long long)n + F;   // inclusive prefix of costs in the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const long long t = __shfl_up(z, off);
        if (lane >= off) z += t;
      }
      int pieces = lane < cnt ? 1 : 0;
      int i0 = 0;           // first request of the chunk not placed yet
      long long zb = 0;     // prefix of costs before request i0
      while (i0 < cnt && p < last) {   // in the last part every request fits whole
        const unsigned long long fit = __ballot(lane >= i0 && lane < cnt && z - zb <= cap);
        const int i1 = i0 + __popcll(fit);   // costs are >= 0: the fitting requests are i0 .. i1 - 1
        if (i1 > i0) {
          const long long zl = readlane64(z, i1 - 1);
          cap -= zl - zb;
          zb = zl;
          i0 = i1;
          if (i0 >= cnt) break;
        }
        // request i0 does not fit whole in what part p has left
        const int n0 = __builtin_amdgcn_readlane(n, i0);
        const long long take = cap - F;
        const int b0 = take > 0 ? (int)take : 0;   // its blocks in part p (take < n0 here)
        const int pi0 = take > 0 ? 1 : 0;
        const int rem = n0 - b0;
        int k = 0;                                 // fresh parts it fills whole
        if (p + 1 < last && rem > D) k = min((int)((unsigned)(rem - 1) / (unsigned)D), last - p - 1);
        for (int j = lane; j <= k; j += 64) {      // parts p + 1 .. p + 1 + k begin inside it
          pb_req[p + 1 + j] = base + i0;
          pb_blk[p + 1 + j] = b0 + j * (int)D;
          pb_piece[p + 1 + j] = pi0 + j;
          pb_n[p + 1 + j] = n0;
        }
        p += 1 + k;
        cap = P - F - (rem - (long long)k * D);    // after its last piece, in part p
        const int pc = pi0 + k + 1;
        if (lane == i0) pieces = pc;
        max_pieces = max(max_pieces, pc);
        zb = readlane64(z, i0);
        ++i0;
      }
      int s = pieces;       // num_splits: inclusive prefix of pieces
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(s, off);
        if (lane >= off) s += t;
      }
      if (lane < cnt) num_splits[base + lane + 1] = acc + s;
      acc += __builtin_amdgcn_readlane(s, 63);
    }
    if (lane == 0) {
      walk_out[0] = p + 1;
      walk_out[1] = max_pieces;
    }
  }
  __syncthreads();
  const int np = walk_out[0];   // parts the walk used
  const int max_pieces = walk_out[1];
  // Rows, one thread per part.  The lengths and block ids a row may need are
  // read together (indices clamped; unused values are ignored), one round
  // trip for all of them.
  for (int q = threadIdx.x; q < num_parts; q += kPlanWaves * 64) {
    int br = 1, er = 0, bb = 0, eb = 0, bp = 0, nr = 0, nb = 0;
    bool evened = false;
    if (q < np) {
      br = pb_req[q];
      bb = pb_blk[q];
      bp = pb_piece[q];
      if (q + 1 < np) {   // part q ends where part q + 1 begins
        nr = pb_req[q + 1];
        nb = pb_blk[q + 1];
        er = nb > 0 ? nr : nr - 1;
      } else {
        er = batch - 1;
      }
      if (br == er) {
        // The part holds request r alone: it takes its even share of the run
        // of such parts of r (the host planner's evening pass).  r's pieces
        // fill parts q - bp .. s1 in order; the first belongs to the run if
        // it begins with r, the last (found by bisection: parts begin in
        // non-decreasing request order) if its end is r's end.
        const int r = br;
        int s0 = q - bp;
        if (pb_req[s0] != r) ++s0;
        int lo = q, hi = np;   // pb_req[lo] == r; the last such part is in [lo, hi)
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pb_req[mid] == r) lo = mid; else hi = mid;
        }
        int s1 = lo;
        const bool tail = s1 + 1 < np ? (pb_blk[s1 + 1] == 0 && pb_req[s1 + 1] == r + 1) : r == batch - 1;
        if (!tail) --s1;
        const int start = pb_blk[s0], end = tail ? pb_n[s1] : pb_blk[s1 + 1];
        const int k = s1 - s0 + 1, i = q - s0, base = (end - start) / k, extra = (end - start) % k;
        bb = start + i * base + min(i, extra);
        eb = bb + base + (i < extra ? 1 : 0);
        evened = true;
      }
    }
    const int len_er = seqlens[er < 0 ? 0 : er];
    const int len_br = seqlens[br < batch ? br : batch - 1];
    const int id = (block_table && q < np) ? block_table[(size_t)br * max_blocks + min(bb, max_blocks - 1)] : -1;
    if (q < np && !evened) eb = (q + 1 < np && nb > 0) ? nb : blocks_of(len_er);
    // With a block table: 1 + the block id of the part's first page when its
    // first piece holds a page (and the id lies in the pool), else 0.
    int first_page = 0;
    if (block_table && q < np) {
      const int end = br == er ? eb : blocks_of(len_br);
      if (bb < end && bb < max_blocks && id >= 0 && id < num_blocks) first_page = id + 1;
    }
    int4* row = reinterpret_cast<int4*>(sched + (size_t)q * MLA_SCHED_INTS);
    row[0] = make_int4(br, er, bb, eb);
    row[1] = make_int4(bp, max_pieces, first_page, 0);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace
}  // namespace mla
