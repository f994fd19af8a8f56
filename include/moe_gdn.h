/*
 * moe_gdn.h -- the GatedDeltaNet recurrent-state update of libmoe.
 *
 * 45 of the pages' model's 60 layers are GatedDeltaNet (linear attention);
 * per decoded token each keeps, per head, a 128 x 128 state matrix, 64 heads
 * per layer, updated with three BLAS routines: a scaling, matrix-vector
 * products and a rank-one update ("48GB内存运行397B模型：Flash-Moe的极端量化与SSD
 * 流式加载实践", section "Metal GPU管线：手写Kernel与FMA优化", paragraph on linear
 * attention (GatedDeltaNet); section "可落地参数清单": 64 heads, state
 * dimension 128; flash-moe README translation, "Kiến trúc" and "Kỹ thuật
 * chính").  The update computed, per head and token, in that order, is the
 * gated delta rule (Yang, Kautz and Hatamizadeh, 2024) with the state S a
 * d_v x d_k matrix:
 *
 *     S <- alpha S;   u = S k;   S <- S + beta (v - u) k^T;   o = S q
 *
 * i.e. S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T and
 * o_t = S_t q_t.  q and k enter as given (their projections, short convolution
 * and normalisation precede this step).
 *
 * Conventions as in moe.h: device pointers owned by the caller, `stream` a
 * hipStream_t (NULL = default), arguments checked on the host before anything
 * is enqueued, negative moe_status_t values on error, fp32 throughout.
 */
#ifndef MOE_GDN_H
#define MOE_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * n_tokens consecutive tokens of one sequence through one layer's heads:
 *   n_heads   heads (64 in the pages' model), 1 .. 4096
 *   d_k, d_v  key and value widths; 128 and 128 are built, other sizes return
 *             MOE_ERR_UNSUPPORTED
 *   state     fp32 [n_heads][d_v][d_k], device, 16-byte aligned: read, then
 *             overwritten in place with the state after the last token
 *   q, k      fp32 [n_tokens][n_heads][d_k], device, 16-byte aligned
 *   v         fp32 [n_tokens][n_heads][d_v], device, 4-byte aligned
 *   alpha     fp32 [n_tokens][n_heads], device: the gate (decay), in (0, 1]
 *   beta      fp32 [n_tokens][n_heads], device: the write strength, in [0, 1]
 *   out       fp32 [n_tokens][n_heads][d_v], device, 4-byte aligned: o per token
 *   n_tokens  1 .. 65535; each token uses the state the previous one left
 * The state is read and written once per call, whatever n_tokens.  out must
 * not overlap the state or the inputs.  Each head's rows are independent, so
 * the results do not depend on the launch shape.
 */
int moe_gdn_update(int32_t n_heads, int32_t d_k, int32_t d_v, int32_t n_tokens, float *state, const float *q,
                   const float *k, const float *v, const float *alpha, const float *beta, float *out,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_GDN_H */
