/*
 * kq_bench.h — measurement helper beside the quantizer (libkq_bench.so): a
 * streaming kernel that moves exactly the quantizer's bytes with no arithmetic,
 * so a benchmark can report the practical HBM ceiling of one call at the same
 * size next to the quantizer's own time.  Not part of the quantizer's API.
 *
 * Same calling rules as kq.h: device pointers owned by the caller, work enqueued
 * on `stream`, host-side checks before any HIP call, negative kq_status values
 * on rejection (-1 null, -2 shape, -3 alignment, -7 HIP).
 */
#ifndef KQ_BENCH_H
#define KQ_BENCH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Access designs of kq_bench_stream_design. */
typedef enum {
  KQB_LANE = 0,  /* one unit per lane, grid-stride loop                             */
  KQB_PAIR = 1,  /* two units per lane (u, u + lanes), both loads before any store   */
  KQB_RING = 2,  /* a lane walks its units with the next two units' loads in flight  */
  KQB_READ = 3,  /* the read half alone (64 B per unit; one byte per lane written)   */
  KQB_WRITE = 4  /* the write half alone (16 + 1 B per unit, nothing read)           */
} kqb_design;

/* For each of `units` 64-byte units of x (contiguous), read the 64 bytes and
 * write 16 bytes to q + 16u and one byte to s + u (values derived from the input
 * so the reads cannot be dropped; they mean nothing).  2.53125 bytes moved per
 * bf16 element, as the quantizer moves (KQB_READ and KQB_WRITE move one side).
 *   x       device, 64 * units bytes, 16-byte aligned
 *   q       device, 16 * units bytes, 16-byte aligned
 *   s       device, units bytes
 *   grid    workgroups of 256 threads (1 .. 65535); lanes loop over the units
 *   design  kqb_design
 * Errors: -1 (null), -2 (units < 0 or >= 2^30, bad grid or design), -3 (alignment),
 * -7 (launch). */
int kq_bench_stream_design(const void* x, int64_t units, uint8_t* q, uint8_t* s, int grid,
                           int design, void* stream);

/* kq_bench_stream_design with KQB_LANE. */
int kq_bench_stream(const void* x, int64_t units, uint8_t* q, uint8_t* s, int grid,
                    void* stream);

#ifdef __cplusplus
}
#endif
#endif
