// Dense MLA decode for MI355X (gfx950): the C ABI -- planning, workspace
// sizes, the launches of the split-KV and combine kernels (mla_kernels.h),
// the allocation-free entry point and the benchmark's per-kernel timing.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
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

}  // namespace mla

#include "mla_kernels.h"


using namespace mla;

extern "C" const char* mla_last_error(void) { return g_last_error.c_str(); }

extern "C" int mla_plan(const int32_t* cache_seqlens, int batch, int num_parts, int fixed_overhead,
                        int force_splits, int32_t* sched_out, int max_parts, int32_t* num_splits_out,
                        int* num_parts_out) {
  return plan(cache_seqlens, batch, num_parts, fixed_overhead, force_splits, sched_out, max_parts,
              num_splits_out, num_parts_out);
}

// Planner policy: one part per CU group (a part is `row_groups` workgroups,
// one per CU), and a per-piece overhead F (in 64-token blocks) that prices
// what a piece costs beyond its pages: the Q load and the first page's
// latency in its prologue, the state merge and the output or partial store
// in its epilogue, and for a split request its share of the combine.
// Parts and overhead for a launch geometry (CU count queried if <= 0);
// `wide`: the 128-row kernel runs (R >= 128, or sparse decode above 16 rows).
static int policy_for(const Geometry& g, bool wide, int* num_cus, int* parts, int* F) {
  if (*num_cus <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(num_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return set_error(MLA_ERR_HIP, "mla_get_metadata: cannot query the CU count");
  }
  *parts = *num_cus / g.row_groups;
  if (*parts < 1) *parts = 1;
  // Per-piece overhead in pages (prologue, epilogue, partial write + merge), measured per kernel.  A
  // 128-row piece of two or more row groups writes (and the combine reads) a partial that many times
  // as large, priced at 6 (two row groups: 0.3 % faster steps than at 4 on the ragged MTP workload).
  *F = g.R <= kSmallRows ? 3 : wide ? (g.row_groups >= 2 ? 6 : 4) : 2;
  return MLA_OK;
}

static int policy(const int32_t* seqlens, int batch, int h_q, int s_q, int is_fp8, int* num_cus, int* parts,
                  int* F) {
  if (batch <= 0 || h_q <= 0 || s_q <= 0 || !seqlens || (is_fp8 != 0 && is_fp8 != 1))
    return set_error(MLA_ERR_INVALID, "mla_get_metadata: batch=%d h_q=%d s_q=%d is_fp8=%d seqlens=%p", batch, h_q,
                     s_q, is_fp8, (const void*)seqlens);
  const Geometry g = geometry(h_q, s_q, is_fp8 != 0);
  return policy_for(g, g.R >= kWideRows || (is_fp8 && g.R > kSmallRows), num_cus, parts, F);
}

extern "C" int mla_max_parts(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int is_fp8, int num_cus,
                             int force_splits) {
  int parts, F;
  int rc = policy(cache_seqlens, batch, h_q, s_q, is_fp8, &num_cus, &parts, &F);
  if (rc) return rc;
  if (force_splits <= 0) return parts;
  long long total = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = pages_of(cache_seqlens[b]);
    total += n < 1 ? 1 : (n < force_splits ? n : force_splits);
  }
  return (int)total;
}

extern "C" int mla_get_metadata(const int32_t* cache_seqlens, int batch, int h_q, int s_q, int is_fp8, int num_cus,
                                int force_splits, int32_t* sched_out, int max_parts,
                                int32_t* num_splits_out, int* num_parts_out, int* total_splits_out) {
  int parts, F;
  int rc = policy(cache_seqlens, batch, h_q, s_q, is_fp8, &num_cus, &parts, &F);
  if (rc) return rc;
  if (!total_splits_out) return set_error(MLA_ERR_INVALID, "mla_get_metadata: null total_splits_out");
  rc = plan(cache_seqlens, batch, parts, F, force_splits, sched_out, max_parts, num_splits_out, num_parts_out);
  if (rc) return rc;
  *total_splits_out = num_splits_out[batch];
  return MLA_OK;
}

extern "C" int mla_plan_attach_pages(int32_t* sched, int num_parts, const int32_t* cache_seqlens, int batch,
                                     const int32_t* block_table, int max_blocks_per_seq, int num_blocks) {
  return attach_pages(sched, num_parts, cache_seqlens, batch, block_table, max_blocks_per_seq, num_blocks);
}

extern "C" int mla_get_metadata_device(const int32_t* cache_seqlens_dev, int batch, int h_q, int s_q, int is_fp8,
                                       int num_cus, int32_t* sched_dev, int max_parts, int32_t* num_splits_dev,
                                       const int32_t* block_table_dev, int max_blocks_per_seq, int num_blocks,
                                       int* num_parts_out, void* stream) {
  if (!sched_dev || !num_splits_dev || !num_parts_out)
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_device: null pointer argument");
  if (block_table_dev && (max_blocks_per_seq <= 0 || num_blocks <= 0))
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_device: block table with max_blocks_per_seq=%d num_blocks=%d",
                     max_blocks_per_seq, num_blocks);
  if (batch > kPlanMaxBatch)
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_device: batch=%d > %d", batch, kPlanMaxBatch);
  int parts, F;
  int rc = policy(cache_seqlens_dev, batch, h_q, s_q, is_fp8, &num_cus, &parts, &F);
  if (rc) return rc;
  if (max_parts < parts)
    return set_error(MLA_ERR_CAPACITY, "mla_get_metadata_device: max_parts=%d < %d parts", max_parts, parts);
  if (parts > kPlanMaxParts)
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_device: %d parts > %d", parts, kPlanMaxParts);
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(kPlanWaves * 64), 0, (hipStream_t)stream, cache_seqlens_dev, batch,
                     parts, F,
                     sched_dev, num_splits_dev, block_table_dev, max_blocks_per_seq, num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "mla_get_metadata_device: launch: %s", hipGetErrorString(e));
  *num_parts_out = parts;
  return MLA_OK;
}

// Sparse decode ("[DeepSeek-3] FlashMLA", section 11): the planner walks
// one "request" per (request, query token), whose length is the number of
// entries of its index list that count (the pages' planner counts blocks
// from topk for sparse decode).
extern "C" int mla_max_parts_sparse(int batch, int s_q, int h_q, int num_cus) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0)
    return set_error(MLA_ERR_INVALID, "mla_max_parts_sparse: batch=%d s_q=%d h_q=%d", batch, s_q, h_q);
  const Geometry g = geometry_sparse(h_q);
  int parts, F;
  const int rc = policy_for(g, g.R > kSmallRows, &num_cus, &parts, &F);
  return rc ? rc : parts;
}

extern "C" int mla_get_metadata_sparse(const int32_t* topk_length, int batch, int s_q, int h_q, int topk,
                                       int num_cus, int32_t* sched_out, int max_parts, int32_t* num_splits_out,
                                       int* num_parts_out, int* total_splits_out) {
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || topk <= 0 || (long long)batch * s_q > (1 << 30))
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_sparse: batch=%d s_q=%d h_q=%d topk=%d", batch, s_q, h_q,
                     topk);
  if (!sched_out || !num_splits_out || !num_parts_out || !total_splits_out)
    return set_error(MLA_ERR_INVALID, "mla_get_metadata_sparse: null pointer argument");
  const Geometry g = geometry_sparse(h_q);
  int parts, F;
  int rc = policy_for(g, g.R > kSmallRows, &num_cus, &parts, &F);
  if (rc) return rc;
  const int n = batch * s_q;
  std::vector<int32_t> lens(n);
  for (int b = 0; b < batch; ++b) {
    const int L = topk_length ? std::min(std::max(topk_length[b], 0), topk) : topk;
    for (int s = 0; s < s_q; ++s) lens[(size_t)b * s_q + s] = L;
  }
  rc = plan(lens.data(), n, parts, F, 0, sched_out, max_parts, num_splits_out, num_parts_out);
  if (rc) return rc;
  *total_splits_out = num_splits_out[n];
  return MLA_OK;
}

extern "C" size_t mla_workspace_bytes(int total_splits, int h_q, int s_q) {
  if (total_splits <= 0 || h_q <= 0 || s_q <= 0) return 0;
  const size_t rows = (size_t)total_splits * h_q * s_q;
  return align256(rows * kDv * sizeof(float)) + align256(rows * sizeof(float));
}

// Kernel timing for mla_profile_start / mla_profile_stop (benchmarks only):
// the kernels are launched with start/stop events attached to their own
// dispatch, so the measured time is the kernel's execution alone.
namespace mla {
namespace {
struct Profile {
  bool on = false;
  int cap = 0, used = 0;
  std::vector<hipEvent_t> ev;  // 4 per call: main start, main stop, combine start, combine stop
};
Profile g_prof;
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};   // checked without the lock by every decode call
}  // namespace
}  // namespace mla

extern "C" int mla_profile_start(int max_calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (max_calls <= 0 || g_prof.on)
    return set_error(MLA_ERR_INVALID, "mla_profile_start: max_calls=%d on=%d", max_calls, (int)g_prof.on);
  g_prof.ev.assign((size_t)max_calls * 4, nullptr);
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) {
      for (auto c : g_prof.ev)
        if (c) (void)hipEventDestroy(c);
      g_prof.ev.clear();
      return set_error(MLA_ERR_HIP, "mla_profile_start: hipEventCreate failed");
    }
  g_prof.cap = max_calls;
  g_prof.used = 0;
  g_prof.on = true;
  g_prof_on.store(true, std::memory_order_release);
  return MLA_OK;
}

extern "C" int mla_profile_stop(float* main_ms, float* combine_ms, int* calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on || !main_ms || !combine_ms || !calls)
    return set_error(MLA_ERR_INVALID, "mla_profile_stop: not started or null output");
  float a = 0.f, c = 0.f;
  int rc = MLA_OK;
  if (g_prof.used > 0 && hipEventSynchronize(g_prof.ev[(size_t)g_prof.used * 4 - 1]) != hipSuccess)
    rc = set_error(MLA_ERR_HIP, "mla_profile_stop: hipEventSynchronize failed");
  for (int i = 0; rc == MLA_OK && i < g_prof.used; ++i) {
    float t0 = 0.f, t1 = 0.f;
    if (hipEventElapsedTime(&t0, g_prof.ev[i * 4], g_prof.ev[i * 4 + 1]) != hipSuccess ||
        hipEventElapsedTime(&t1, g_prof.ev[i * 4 + 2], g_prof.ev[i * 4 + 3]) != hipSuccess)
      rc = set_error(MLA_ERR_HIP, "mla_profile_stop: hipEventElapsedTime failed");
    a += t0;
    c += t1;
  }
  *main_ms = a;
  *combine_ms = c;
  *calls = g_prof.used;
  for (auto e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.on = false;
  g_prof_on.store(false, std::memory_order_release);
  return rc;
}

static hipEvent_t* profile_slot() {
  if (!g_prof_on.load(std::memory_order_acquire)) return nullptr;   // the decode path: no lock when off
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on || g_prof.used >= g_prof.cap) return nullptr;
  return &g_prof.ev[(size_t)(g_prof.used++) * 4];
}

constexpr int kCombineMaxGrid = 8192;   // about four rounds of resident workgroups (measured: 2048 left the
                                         // 32768 pairs of workload 4 at four serial round trips a wave, 14 % slower)

// Enqueues the split-KV kernel picked by the row count (and, for sparse
// decode or an FP8 cache, its variant), then the combine kernel.  Sparse
// decode and FP8 caches take the 128-row kernel above 16 rows.
template <bool kSparse, bool kFp8>
static const void* pick_main_kernel(const Geometry& g) {
  if (g.R <= kSmallRows) return (const void*)mla_splitkv_small_kernel<kSparse, kFp8>;
  // Row groups of one part share pages through L2 (cached copies); a single
  // group streams every page once (nontemporal copies).
  return g.row_groups == 1 ? (const void*)mla_splitkv_wide_kernel<true, kSparse, kFp8>
                           : (const void*)mla_splitkv_wide_kernel<false, kSparse, kFp8>;
}

// The small-row kernel's split partials (fp32, 2 KB a row) go out with the
// nontemporal hint only when there are many of them: written as plain stores
// they wait in L2 for the end-of-kernel write-back, which costs more than the
// combine then saves on reading them once they are megabytes (memory-bound
// workload, ~7.7 MB at most: 17.7 us a step either way, within 0.1-0.3 us, in
// A/Bs on one GPU), while a few hundred KB are written back quickly and read
// sooner (tiny workload, 0.26 MB: 9.1 against 9.5 us a step bf16, 9.3 against
// 9.8 us FP8).  The bound is the slots the plan can fill (parts + batch - 1).
constexpr size_t kNtPartialBytes = 1u << 20;

static int launch_decode(Params& prm, Geometry g, bool sparse, bool fp8, hipStream_t st, const char* who) {
  hipEvent_t* ev = profile_slot();
  const void* main_fn;
  prm.row_groups = g.row_groups;
  prm.nt_partials = (size_t)(prm.num_parts + prm.batch - 1) * g.R * kDv * sizeof(float) > kNtPartialBytes ? 1 : 0;
  // (the leading scalar arguments: MLA_SPLITKV_HOT_ARGS, then Params)
  void* args[] = {&prm.sched,   &prm.num_parts,  &prm.row_groups, &prm.max_blocks, &prm.block_table,
                  &prm.seqlens, &prm.num_splits, &prm.kv,         &prm.q,          &prm};
  // (MLA_COMBINE_HOT_ARGS, then Params)
  void* cargs[] = {&prm.sched, &prm.num_splits, &prm.batch, &prm.R, &prm.lacc, &prm.oacc, &prm};
  // The XCD-aware block mapping (map_block) needs 8 * row_groups * ceil(parts / 8) workgroups.
  const int grid = 8 * g.row_groups * ((prm.num_parts + 7) / 8);
  if (g.R > kSmallRows && g.R < kWideRows && !sparse && !fp8)
    main_fn = (const void*)mla_splitkv_kernel;
  else if (sparse)
    main_fn = fp8 ? pick_main_kernel<true, true>(g) : pick_main_kernel<true, false>(g);
  else
    main_fn = fp8 ? pick_main_kernel<false, true>(g) : pick_main_kernel<false, false>(g);
  // Plain launches unless profiling (these are what stream capture records).
  hipError_t e = ev ? hipExtLaunchKernel(main_fn, dim3(grid), dim3(256), args, 0, st, ev[0], ev[1], 0)
                    : hipLaunchKernel(main_fn, dim3(grid), dim3(256), args, 0, st);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "%s: main kernel launch: %s", who, hipGetErrorString(e));
  const long long pairs = (long long)prm.batch * g.R;
  const int cgrid = (int)(pairs < kCombineMaxGrid ? pairs : kCombineMaxGrid);
  e = ev ? hipExtLaunchKernel((const void*)mla_combine_kernel, dim3(cgrid), dim3(kCombineWaves * 64), cargs, 0, st,
                              ev[2], ev[3], 0)
         : hipLaunchKernel((const void*)mla_combine_kernel, dim3(cgrid), dim3(kCombineWaves * 64), cargs, 0, st);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "%s: combine launch: %s", who, hipGetErrorString(e));
  return MLA_OK;
}

extern "C" int mla_decode_fwd(const void* q, const void* kv_cache, const int32_t* block_table,
                              const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_blocks,
                              int max_blocks_per_seq, float softmax_scale, int causal, int is_fp8,
                              const int32_t* sched, int num_parts, const int32_t* num_splits, void* workspace,
                              size_t workspace_bytes, void* out, float* lse, void* stream) {
  if (!q || !kv_cache || !block_table || !cache_seqlens || !sched || !num_splits || !out || !lse)
    return set_error(MLA_ERR_INVALID, "mla_decode_fwd: null pointer argument");
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || num_parts <= 0)
    return set_error(MLA_ERR_INVALID,
                     "mla_decode_fwd: batch=%d s_q=%d h_q=%d num_blocks=%d max_blocks_per_seq=%d num_parts=%d",
                     batch, s_q, h_q, num_blocks, max_blocks_per_seq, num_parts);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return set_error(MLA_ERR_INVALID, "mla_decode_fwd: softmax_scale must be finite and >= 0");
  if (causal != 0 && causal != 1) return set_error(MLA_ERR_INVALID, "mla_decode_fwd: causal must be 0 or 1");
  if (is_fp8 != 0 && is_fp8 != 1) return set_error(MLA_ERR_INVALID, "mla_decode_fwd: is_fp8 must be 0 or 1");
  const Geometry g = geometry(h_q, s_q, is_fp8 != 0);
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
  const size_t rows = (size_t)slots * g.R;
  prm.oacc = (float*)workspace;
  prm.lacc = (float*)((char*)workspace + align256(rows * kDv * sizeof(float)));
  prm.batch = batch;
  prm.R = g.R;
  prm.h_q = h_q;
  prm.s_q = s_q;
  prm.max_blocks = max_blocks_per_seq;
  prm.num_parts = num_parts;
  prm.row_groups = g.row_groups;
  prm.causal = causal;
  prm.scale_log2 = softmax_scale * kLog2e;
  prm.indices = nullptr;
  prm.topk_len = nullptr;
  prm.topk = 0;
  prm.kv_tokens = num_blocks * kPage;
  prm.fold = 1;

  return launch_decode(prm, g, false, is_fp8 != 0, (hipStream_t)stream, "mla_decode_fwd");
}

// ---------------------------------------------------------------------------
// Split workspace owned by the library, for callers that cannot allocate
// (mla_decode_fwd_noalloc).  One copy per GPU, placed when the code object is
// loaded on that GPU and held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace mla {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch` (looked up on first use).
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MLA_ERR_HIP, "mla_decode_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MLA_ERR_INVALID, "mla_decode_fwd_noalloc: device %d >= %d", dev, kMaxDevices);
  void* ptr = g_scratch_dev[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ptr = g_scratch_dev[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return set_error(MLA_ERR_HIP, "mla_decode_fwd_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                         hipGetErrorString(e));
      g_scratch_dev[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MLA_OK;
}
}  // namespace
}  // namespace mla

extern "C" int mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                      const int32_t* cache_seqlens, int batch, int s_q, int h_q, int num_blocks,
                                      int max_blocks_per_seq, float softmax_scale, int causal, int is_fp8,
                                      const int32_t* sched, int num_parts, const int32_t* num_splits, void* out,
                                      float* lse, void* stream) {
  // Size check first (host arithmetic only; invalid sizes give 0 here and are
  // reported by mla_decode_fwd's own checks).
  const size_t need = (batch > 0 && num_parts > 0) ? mla_workspace_bytes(num_parts + batch - 1, h_q, s_q) : 0;
  if (need > kNoAllocScratchBytes)
    return set_error(MLA_ERR_WORKSPACE,
                     "mla_decode_fwd_noalloc: this plan needs %zu bytes of split workspace > the library's %zu "
                     "(use mla_decode_fwd with a caller workspace)",
                     need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  return mla_decode_fwd(q, kv_cache, block_table, cache_seqlens, batch, s_q, h_q, num_blocks, max_blocks_per_seq,
                        softmax_scale, causal, is_fp8, sched, num_parts, num_splits, ws, kNoAllocScratchBytes, out,
                        lse, stream);
}

extern "C" int mla_decode_sparse_fwd(const void* q, const void* kv_cache, const int32_t* indices,
                                     const int32_t* topk_length, int batch, int s_q, int h_q, int num_blocks,
                                     int topk, float softmax_scale, int is_fp8, const int32_t* sched, int num_parts,
                                     const int32_t* num_splits, void* workspace, size_t workspace_bytes, void* out,
                                     float* lse, void* stream) {
  if (!q || !kv_cache || !indices || !sched || !num_splits || !out || !lse)
    return set_error(MLA_ERR_INVALID, "mla_decode_sparse_fwd: null pointer argument");
  if (batch <= 0 || s_q <= 0 || h_q <= 0 || num_blocks <= 0 || num_blocks > (1 << 24) || topk <= 0 ||
      num_parts <= 0 || (long long)batch * s_q > (1 << 30))
    return set_error(MLA_ERR_INVALID, "mla_decode_sparse_fwd: batch=%d s_q=%d h_q=%d num_blocks=%d topk=%d num_parts=%d",
                     batch, s_q, h_q, num_blocks, topk, num_parts);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return set_error(MLA_ERR_INVALID, "mla_decode_sparse_fwd: softmax_scale must be finite and >= 0");
  if (is_fp8 != 0 && is_fp8 != 1) return set_error(MLA_ERR_INVALID, "mla_decode_sparse_fwd: is_fp8 must be 0 or 1");
  const Geometry g = geometry_sparse(h_q);
  const int n = batch * s_q;   // one split-KV "request" per (request, query token)
  const int slots = num_parts + n - 1;
  const size_t need = mla_workspace_bytes(slots, h_q, 1);
  if (!workspace || workspace_bytes < need)
    return set_error(MLA_ERR_WORKSPACE, "mla_decode_sparse_fwd: workspace %zu bytes < %zu needed", workspace_bytes,
                     need);
  Params prm;
  prm.q = (const unsigned char*)q;
  prm.kv = (const unsigned char*)kv_cache;
  prm.block_table = nullptr;
  prm.seqlens = nullptr;
  prm.sched = sched;
  prm.num_splits = num_splits;
  prm.out = (unsigned short*)out;
  prm.lse = lse;
  const size_t rows = (size_t)slots * g.R;
  prm.oacc = (float*)workspace;
  prm.lacc = (float*)((char*)workspace + align256(rows * kDv * sizeof(float)));
  prm.batch = n;
  prm.R = g.R;
  prm.h_q = h_q;
  prm.s_q = 1;
  prm.max_blocks = 1;
  prm.num_parts = num_parts;
  prm.row_groups = g.row_groups;
  prm.causal = 0;
  prm.scale_log2 = softmax_scale * kLog2e;
  prm.indices = indices;
  prm.topk_len = topk_length;
  prm.topk = topk;
  prm.kv_tokens = num_blocks * kPage;
  prm.fold = s_q;
  return launch_decode(prm, g, true, is_fp8 != 0, (hipStream_t)stream, "mla_decode_sparse_fwd");
}

