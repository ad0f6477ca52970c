/*
 * gdn_bench.h - measurement kernels that sit beside libgdn.so (built into
 * libgdn_bench.so).  Not part of the GDN step: they give the benchmark a
 * measured ceiling for the step's memory traffic on the same GPU.
 */
#ifndef GDN_BENCH_H
#define GDN_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gdn_bench_state_fanout - the SSM-state traffic of one spec-verify call and
 * nothing else: for every spec row b and v-head h, the dv*dk fp32 block of
 * v-head h is read from slot spec_state_indices[b][n_acc-1]
 * (zeros for a slot <= 0) and written to slot spec_state_indices[b][t] for
 * each of the row's T_b tokens (slots <= 0 skipped) - the load and the
 * per-token stores of "[GDN] Spec-decoding-aware attention kernel"
 * ("Changes", IS_SPEC slots), with no conv, gates or arithmetic.  Each
 * token's copy has its first element bumped by t, so the stores are not
 * identical.
 *
 *   ssm_state   [num_slots, Hv, dv, dk] fp32, device (read and written)
 *   spec_query_start_loc [num_rows+1], spec_state_indices [num_rows,
 *   max_spec_len], num_accepted_tokens [num_rows]: int32, device
 *   stream: hipStream_t (NULL = default stream)
 *
 * One 512-thread workgroup per (row, v-head), the v-heads of a row on one
 * XCD, one workgroup per CU; each wave instruction moves 1 KiB of
 * consecutive bytes with non-temporal loads and stores (measured on MI355X
 * the fastest of the layouts tried for this traffic: 95.6 us at K=3,
 * batch 64, against 103.4 us with 128 KiB (row, k-head) blocks).  On grids
 * of at least two units per CU the last eighth of the units (at most two
 * per CU) is claimed at run time by the last workgroup of each CU, as in
 * the row kernel, from a wrapping count in the library's own device memory
 * (0 again after every call; calls on one GPU must be ordered).  Supports
 * dv*dk == 16384 (dk = dv = 128).  num_k_heads only checks the shape.
 * Slots, n_acc and T_b are clamped to stay inside the pool.  Returns 0, -1
 * for an unsupported shape or NULL pointer, -7 when the launch fails.
 */
int gdn_bench_state_fanout(float* ssm_state, int32_t num_slots, int32_t num_k_heads,
                           int32_t num_v_heads, int32_t head_k_dim, int32_t head_v_dim,
                           int32_t num_rows, int32_t max_spec_len,
                           const int32_t* spec_query_start_loc,
                           const int32_t* spec_state_indices,
                           const int32_t* num_accepted_tokens, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_BENCH_H */
