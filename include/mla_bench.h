/*
 * mla_bench.h — measurement kernels used by the benchmark, in their own
 * library (libmla_bench.so); the decode library does not use them.
 *
 * They give the two figures a decode kernel's rates are read against: the
 * rate at which the GPU streams a buffer from memory (the attainable read
 * roof, beside the nominal HBM peak), and the fixed cost of one kernel
 * launch (which a split-KV decode pays twice: main kernel and combine).
 * Return 0, or -1 with a message from mla_bench_last_error().
 */
#ifndef MLA_BENCH_H
#define MLA_BENCH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one read of bytes (>= 16; a multiple of 16 is read whole) of the
 * device buffer buf on stream, split over `grid` workgroups of 256 lanes,
 * 16-byte nontemporal loads; sink: device unsigned [grid], written only in a
 * practically impossible case (it keeps the loads from being removed). */
int mla_bench_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream);

/* Enqueue an empty kernel of `grid` workgroups of 256 lanes on stream. */
int mla_bench_empty(int grid, void* stream);

const char* mla_bench_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_BENCH_H */
