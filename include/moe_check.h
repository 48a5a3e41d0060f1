/*
 * moe_check.h -- host-only self-checks of libmoe.so's launch plans.
 *
 * These functions do no GPU work and allocate nothing.  They let a test on a
 * machine without a GPU walk the exact launch shape a kernel would get and
 * confirm that every memory access it makes stays inside the buffer the
 * library sizes for it.  They are not part of the layer.
 */
#ifndef MOE_MI355X_CHECK_H
#define MOE_MI355X_CHECK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The bf16 router gate's launch from a copy of the router weights (made by
 * moe_forward in its workspace: the split copy of bf16 parts where it lets
 * the grid fill the CUs, else the blocked fp32 copy on large gates): for B
 * tokens, hidden size d and E experts, *read_end receives the exclusive
 * end, in bytes, of what the gate kernel would read from that copy, and
 * *copy_bytes the copy's size in the forward's workspace (for the blocked
 * copy when neither is used).  Returns 1 if moe_forward would use the split
 * copy at this shape, 2 the blocked copy, 0 neither (both outputs are
 * filled either way), -1 on bad arguments (B < 1, d < 8 or not a multiple
 * of 8, E < 1 or E > 1024, or a null pointer). */
int32_t moe_check_gate_split_reach(int64_t B, int32_t d, int32_t E, int64_t* read_end,
                                   int64_t* copy_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_CHECK_H */
