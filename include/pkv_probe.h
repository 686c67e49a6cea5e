/*
 * pkv_probe.h - a compute-only timing probe for the decode kernels' inner
 * step, in its own library (libpkv_probe.so), apart from libpkv.so.
 *
 * It is a measurement aid, not part of the attention path: it answers the
 * design question of whether one GQA group's q.K^T and P.V for a 16-token
 * block of one KV head (bf16 K/V, head dim 128) is cheaper on the matrix
 * cores or on the vector ALU.  The pages describe a paged decode kernel
 * that walks a sequence's blocks through its block table and forms each
 * block's attention scores and value sum ([KVP] §三 工作方式, [BJD] §3
 * PagedAttention与分页管理) but say nothing about which execution units
 * compute them; the probe times both ways on gfx950 with no HBM traffic, so
 * the per-block compute time can be set against the time the same block
 * takes to stream from HBM.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `workgroups` workgroups of four 64-lane waves (one wave per SIMD,
 * as the decode kernel runs); each wave loops over `chunks` 16-token blocks
 * whose K and V words change every iteration, computing per block:
 *   variant 0  only the per-block operand changes and loop control both
 *              compute variants carry (the floor to subtract);
 *   variant 1  matrix cores: the 16 query columns' logits with four
 *              v_mfma_f32_16x16x32_bf16, the streaming-softmax update, and
 *              P.V with sixteen v_mfma_f32_16x16x16_bf16 (p as a bf16 hi + lo
 *              pair), the decode kernel's own arithmetic;
 *   variant 2  vector ALU, 8 query heads per KV head (the 70B shape):
 *              logits with v_dot2_f32_bf16 on each lane's 32 dims and a
 *              four-lane sum, the same softmax update, p gathered from the
 *              lanes of its tokens and P.V with v_dot2_f32_bf16 (hi + lo);
 *   variant 3  as variant 2 with 4 query heads per KV head (the 8B shape).
 * seed: device pointer to 4096 32-bit words, each two bf16 values that are
 *       finite; they seed K, V and q (lane l reads words 64 l .. 64 l + 63).
 * out:  device pointer to workgroups * 256 floats, written (one sum per
 *       lane, kept so the compiler drops nothing; its value has no meaning).
 * chunks >= 0, 1 <= workgroups <= 65536.
 * Returns hipSuccess (0) or the hipError_t of a bad argument or of the
 * launch; asynchronous on `stream` like every launch. */
int pkv_probe_compute(int variant, const uint32_t* seed, float* out, int chunks, int workgroups,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
