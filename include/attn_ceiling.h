/*
 * attn_ceiling.h - C ABI of libattn_ceiling.so, a measurement probe for
 * AMD Instinct MI355X (gfx950) that sits beside libattn.so. It is not part
 * of the attention computation.
 *
 * What it measures. The sustained rate of the matrix cores (32x32x16 bf16
 * products, 256 workgroups of 8 waves, two waves per SIMD on every CU) when
 * every 8 products are interleaved with the vector-ALU and LDS instructions
 * one attention kernel issues per 8 products: its exponentials, its other
 * vector instructions and its 16-byte and 8-byte LDS operand reads (counts
 * taken from the kernels' instruction counters). There is no global memory
 * traffic, no barrier and no dependency between the vector work and the
 * products, so the rate bounds any kernel with that instruction mix from
 * above. Operands are random bf16 values, except for ATTN_MIX_CONSTANT:
 * the matrix cores draw more power, and run slower, on random data.
 *
 * Reading a roofline. The attention kernels' matrix-core throughput divided
 * by the ceiling of their own mix says how much of what that mix allows they
 * reach; divided by the published 2.5 PFLOP/s bf16 peak it says how far the
 * chip's nominal rate is.
 */
#ifndef ATTN_CEILING_H
#define ATTN_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Instruction mixes, per 8 products: vector-ALU instructions (all but the
 * products themselves; of them exponentials), 16-byte and 8-byte LDS reads.
 * The totals equal the kernels' SQ_INSTS_VALU (less their products),
 * SQ_INSTS_VALU_TRANS_F32 and SQ_INSTS_LDS counts per product, x 8. */
enum {
  ATTN_MIX_CONSTANT = 0, /* products only, constant operands                          */
  ATTN_MIX_RANDOM = 1,   /* products only, random operands                            */
  ATTN_MIX_DKDV = 2,     /* dK/dV kernels, d_k = 64:   36 VALU (8 exp),  8 + 8 LDS   */
  ATTN_MIX_DQ = 3,       /* dQ kernel, d_k = 64:       40 VALU (11 exp), 2 + 4 LDS   */
  ATTN_MIX_FWD64 = 4,    /* forward, d_k = 64:         54 VALU (16 exp), 4 + 8 LDS   */
  ATTN_MIX_FWD128 = 5    /* forward, d_k = 128:        26 VALU (8 exp),  4 + 8 LDS   */
};

/* Device workspace the probe needs (random operands, LDS contents, outputs). */
size_t attn_mix_ceiling_workspace_bytes(void);

/* FLOP of one probe launch with `iters` iterations (8 products each per wave). */
double attn_mix_ceiling_flop(int iters);

/*
 * Fills `workspace` (device memory, 16-byte aligned, owned by the caller, at
 * least attn_mix_ceiling_workspace_bytes()) with random operands, runs three
 * untimed and ten timed launches of the probe for `mix` on `stream` (a
 * hipStream_t, NULL = default stream), waits for them and stores the average
 * launch time in *ms (host pointer). The rate is attn_mix_ceiling_flop(iters)
 * / *ms. Blocks until the timed launches finish.
 * Returns 0, -1 (unknown mix, iters < 1, null or misaligned pointer), -3
 * (workspace too small) or -4 (the HIP runtime rejected a launch or event).
 */
int attn_mix_ceiling(int mix, int iters, void* workspace, size_t workspace_bytes, float* ms, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CEILING_H */
