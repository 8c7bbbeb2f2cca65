/* Spatial SwiGLU block of a GTR layer, forward pass, on one AMD MI355X (gfx950).
 *
 * What it computes.  Every GTR layer pairs the gated-linear-attention token
 * mixer (gtr_gla.h) with a Spatial SwiGLU block that mixes neighbouring
 * positions: SwiGLU with a 3 x 3 per-channel convolution in its value branch
 * (x-techcon article on GTR, section 架构 / Architecture; the abstract page
 * calls these "spatially enhanced SwiGLU blocks").  The pages say nothing more,
 * so this library reads it as
 *
 *   u   = x W_in                       (W_in = [W_g | W_v], C x 2F)
 *   h   = SiLU(u_g) * (DWConv3x3(u_v) + b)
 *   out = h W_out                      (F x C)
 *
 * with the convolution a per-channel cross-correlation over the patch grid:
 * tap (dy, dx) multiplies the value at (row + dy - 1, col + dx - 1), zero
 * outside the grid.  No normalisation or residual (those belong to the layer).
 *
 * Layouts (all row-major, dense, one element type = the I/O dtype):
 *   x, out  : [B][grid_h][grid_w][C]
 *   w_in    : [C][2F], gate projection in columns [0, F), value in [F, 2F)
 *   conv_w  : [3][3][F], taps first, channels contiguous
 *   conv_b  : [F], or NULL for no bias
 *   w_out   : [F][C]
 * Arithmetic: the projections are library GEMMs (rocBLAS) with fp32
 * accumulation; u is kept in fp16 for fp16 I/O and in fp32 otherwise; h is
 * rounded to the I/O dtype before the output projection, except for bf16 I/O,
 * where h is fp16 and W_out is converted to fp16 for the projection (so |h|
 * and |W_out| must stay below 65504; W_out loses bits only below 2^-17),
 * whose fp32 result is then rounded; out is rounded to the I/O dtype.
 *
 * Ownership and errors as in gtr_gla.h: device pointers owned by the caller,
 * 16-byte aligned; out must not overlap an input; the library owns a
 * per-(device, stream) workspace (u and h) that is grown outside stream
 * capture only (GTR_ERR_CAPTURE otherwise: run the shape once eagerly first)
 * and freed by gtr_gla_release_workspaces();
 * errors are negative GTR_ERR_* codes with a message from gtr_gla_last_error().
 * Sizes: C and F multiples of 8 from 8 to 65536, 0 <= B*grid_h*grid_w <= 2^24.
 * A call with no tokens returns GTR_OK and touches nothing.
 */
#ifndef GTR_SWIGLU_H
#define GTR_SWIGLU_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#include "gtr_gla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out = Spatial SwiGLU(x), asynchronous on `stream`.  dtype: GTR_DTYPE_F32,
 * GTR_DTYPE_F16 or GTR_DTYPE_BF16.  Returns GTR_OK or a GTR_ERR_* code;
 * GTR_ERR_LAUNCH also covers a failed library GEMM. */
int gtr_swiglu_fwd(const void *x, const void *w_in, const void *conv_w, const void *conv_b,
                   const void *w_out, void *out, int B, int grid_h, int grid_w, int C, int F,
                   int dtype, hipStream_t stream);

/* Workspace bytes the library keeps for a shape (0 for an invalid or empty one). */
size_t gtr_swiglu_workspace_bytes(int B, int grid_h, int grid_w, int C, int F, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* GTR_SWIGLU_H */
