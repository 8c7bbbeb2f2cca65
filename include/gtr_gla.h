/*
 * gtr_gla.h - C ABI of the MI355X (gfx950) chunkwise forward pass of
 * key-only-gated linear attention (GLA), the token mixer of GTR (Gated Token
 * Recurrence).
 *
 * What every entry point computes
 * -------------------------------
 * Source: x-techcon article on GTR ("视觉AI看得越细，还能又快又准吗？..."),
 * section 架构 (Architecture), and the abstract of "GTR: Gated Token
 * Recurrence for Efficient Dense Prediction" (goodpapers.org listing).
 * For each sequence (b, h) the patch grid of grid_h x grid_w tokens is visited
 * in one of four scan orders.  A d_k x d_v state S starts at zero (or at a
 * caller-supplied S_0) and, at each scan position t,
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t ,  alpha_t = exp(log_gate_t),
 *     o_t = q_t S_t ,
 * i.e. the state first decays per KEY dimension by an input-generated gate
 * (the value-side decay is 1), then takes the current key/value outer
 * product, and the query reads the UPDATED state.  The article's printed
 * formula did not survive extraction; the sentences around it fix the
 * reading above.  No q.k scale and no softmax are applied.
 *
 * Scan orders (same section; the article names them, the index formulas are
 * this library's reading): with grid cells numbered row-major n = r*grid_w + c
 * and N = grid_h*grid_w,
 *   GTR_DIR_L2R = 0  n(t) = t                         (row-major)
 *   GTR_DIR_R2L = 1  n(t) = N-1-t                     (L->R reversed)
 *   GTR_DIR_T2B = 2  n(t) = (t % grid_h)*grid_w + t / grid_h   (column-major)
 *   GTR_DIR_B2T = 3  n(t) = n_T2B(N-1-t)              (T->B reversed)
 * Every output is written back at the grid position of its own token (the
 * scan order only decides which tokens precede it), so out has the layout of
 * the inputs.
 *
 * How: the operator section of the same article splits the scan into
 * 64-token chunks, computes each chunk's state contribution in parallel,
 * passes chunk-boundary states along, then forms each chunk's outputs in
 * parallel.  This library does the same with hand-written gfx950 kernels
 * (MFMA contractions, scores kept in LDS); the result does not depend on the
 * chunking beyond floating-point rounding.
 *
 * Layout (all tensors dense, row-major, one element type per call):
 *   q, k, log_gate : [B][H][grid_h][grid_w][d_k]
 *   v, out         : [B][H][grid_h][grid_w][d_v]
 *   s0, s_final    : [B][H][d_k][d_v] float32 (entry point _ex only)
 * log_gate holds natural-log alpha; finite values <= 0 are the domain
 * (log-sigmoid outputs).  Outside it the output is unspecified.
 *
 * Ownership and execution:
 *   - All tensor pointers are caller-owned memory of the current HIP device.
 *     The library never frees them.  out must not overlap any input.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  The library
 *     keeps one internal workspace per (device, stream); it is allocated on
 *     first use and grown when a larger call arrives.  Growing it is refused
 *     while `stream` is being captured into a graph (GTR_ERR_CAPTURE): make
 *     one call of the largest shape before capturing.  Calls on one stream
 *     are ordered by that stream; calls on different streams use different
 *     workspaces.  A graph captured from a stream uses that stream's
 *     workspace, so replay it only where a call on that stream could run:
 *     not beside another call on that stream or another replay of a graph
 *     captured from it.  A workspace that grows keeps its old buffers until
 *     gtr_gla_release_workspaces(), so graphs captured earlier stay valid.
 *   - Every argument is validated on the host before the first HIP call;
 *     a call that returns an error has launched nothing.  Outside stream
 *     capture each pointer is also checked to be device memory of the
 *     current device with room for its tensor (GTR_ERR_POINTER); while the
 *     stream is being captured that query is skipped, so capture a call only
 *     after the same call has run eagerly.  Faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Four environment variables serve tests and measurement only:
 *     GTR_GLA_SKIP_POINTER_CHECKS=1 skips the device-pointer queries,
 *     GTR_GLA_TEST_FAIL_ALLOC=1 makes every workspace allocation fail
 *     (GTR_ERR_ALLOC), which leaves the caches as they were,
 *     GTR_GLA_FOLD_BLOCK=n (1..32) sets how many segments the one-launch path
 *     groups into a fold block, and GTR_GLA_SCAN=lanes runs boundary scans of
 *     at most 64 steps as scans across the lanes of a wave (slower; read at
 *     every call).  Results change only by rounding.
 *
 * Supported sizes: d_k and d_v multiples of 4 from 4 to 128 (64 is the tuned
 * case); 0 <= grid_h*grid_w <= 2^23 and
 * grid_h*grid_w*max(d_k, d_v)*element bytes <= 2^31; 0 <= B*H <= 2^20; and
 * the launch grids fit 31 bits: B*H*ceil(d_v/64)*ceil(d_k/64) times the
 * segments per sequence (forward) or the 64-token chunks per sequence
 * (backward) at most 2^31 - 1 (GTR_ERR_INVALID_ARG otherwise).
 * Pointers must be 16-byte aligned.
 *
 * Value range.  For fp16 and bf16 I/O the matrix operands are fp16 (products
 * accumulate in fp32), so whatever becomes an operand must stay within the
 * fp16 range, |x| <= 65504:
 *   - the inputs themselves (bf16 values beyond it become infinite);
 *   - q and k times at most 2^8, on the within-chunk diagonal score tiles
 *     (|q|, |k| < 256 always suffices there);
 *   - each within-chunk score, which is at most |q_t|*|k_s| (Euclidean norms
 *     of a query and an earlier key of the same chunk).
 * Beyond these the output is unspecified (typically inf or NaN).  The state,
 * kept in fp32, is not limited by this: it becomes an operand only after an
 * exact power of two brings its largest entry near 2^14.  fp32 I/O uses fp32
 * operands throughout and has none of these limits.
 *
 * Empty calls: with B*H == 0 or no tokens there is nothing to compute and
 * tensor pointers may be NULL; the call returns GTR_OK without touching the
 * device, except that with tokens == 0, B*H > 0 and s_final given, s_final
 * receives s0 (or zeros) - the state after an empty scan is the state before.
 */
#ifndef GTR_GLA_H
#define GTR_GLA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* scan directions */
#define GTR_DIR_L2R 0
#define GTR_DIR_R2L 1
#define GTR_DIR_T2B 2
#define GTR_DIR_B2T 3

/* element types of q, k, v, log_gate and out */
#define GTR_DTYPE_F32 0
#define GTR_DTYPE_F16 1
#define GTR_DTYPE_BF16 2

/* launch structure (entry points _ex, _check, _workspace_bytes, _plan) */
#define GTR_PATH_AUTO 0   /* chosen by the library from the shape */
#define GTR_PATH_FUSED 1  /* one kernel: segment aggregates, a fixed-order fold within blocks of
                             segments and a chain between blocks, outputs */
#define GTR_PATH_SPLIT 2  /* three kernels: segment aggregates, boundary scan, outputs */

/* return codes: 0 on success, negative on error */
#define GTR_OK 0
#define GTR_ERR_INVALID_ARG (-1)  /* null pointer, negative or too large size, bad direction/dtype/path */
#define GTR_ERR_UNSUPPORTED (-2)  /* d_k or d_v above 128 or not a multiple of 4 */
#define GTR_ERR_ALIGNMENT (-3)    /* a pointer is not 16-byte aligned */
#define GTR_ERR_ALIAS (-4)        /* out (or s_final) overlaps an input */
#define GTR_ERR_NO_DEVICE (-5)    /* no usable HIP device */
#define GTR_ERR_POINTER (-6)      /* a pointer is not device memory of the current device,
                                     or its allocation is smaller than the tensor */
#define GTR_ERR_ALLOC (-7)        /* workspace allocation failed */
#define GTR_ERR_CAPTURE (-8)      /* workspace would have to grow during stream capture */
#define GTR_ERR_LAUNCH (-9)       /* a kernel launch failed */
#define GTR_ERR_TIMEOUT (-10)     /* a one-launch-path wait between workgroups gave up (see gtr_gla_stream_status) */
#define GTR_ERR_SCRATCH (-11)     /* gtr_gla_fwd_static: the shape needs more working memory than its fixed array */

/*
 * Generic entry point: dtype selects the element type (GTR_DTYPE_*).
 * Arguments: q, k, v, log_gate (inputs), out (output), B batch, H heads,
 * grid_h x grid_w patch grid, d_k key width, d_v value width, direction
 * (GTR_DIR_*), stream.
 */
int gtr_gla_fwd(const void *q, const void *k, const void *v, const void *log_gate,
                void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                int direction, int dtype, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): gtr_gla_fwd with the
 * same arguments and results, computed by the three-launch path, whose only
 * working memory (the boundary states) comes from a fixed array in the
 * library's device code: GTR_GLA_STATIC_SCRATCH_BYTES per device, held from
 * the library's load until the process ends.  It calls no hipMalloc or hipFree
 * and nothing that allocates.  The segment length is the library's choice,
 * lengthened up to 32 chunks if the states would not fit; a shape that still
 * does not fit returns GTR_ERR_SCRATCH with a message (e.g. one 2^23-token
 * sequence; any number of sequences of at most 32 chunks always fits).  Every
 * call on a device shares that device's array: calls that overlap on one
 * device (other streams or threads, graph replays) race and give undefined
 * outputs.  Each call writes every word it reads, so no clearing is needed.
 */
#define GTR_GLA_STATIC_SCRATCH_BYTES (32u << 20)
int gtr_gla_fwd_static(const void *q, const void *k, const void *v, const void *log_gate,
                       void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                       int direction, int dtype, hipStream_t stream);

/* Typed entry points with the plain argument list; the element type is in the name. */
int gtr_gla_fwd_f32(const void *q, const void *k, const void *v, const void *log_gate,
                    void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                    int direction, hipStream_t stream);
int gtr_gla_fwd_f16(const void *q, const void *k, const void *v, const void *log_gate,
                    void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                    int direction, hipStream_t stream);
int gtr_gla_fwd_bf16(const void *q, const void *k, const void *v, const void *log_gate,
                     void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                     int direction, hipStream_t stream);

/*
 * Extended entry point.  Same recurrence, plus:
 *   s0       (nullable) float32 [B][H][d_k][d_v], the state before the first
 *            scan position (NULL = zero state);
 *   s_final  (nullable) float32 [B][H][d_k][d_v], receives the state after the
 *            last scan position (NULL = not wanted);
 *   chunks_per_segment  how many consecutive 64-token chunks one workgroup
 *            walks with its state held in registers (<= 0 = chosen by the
 *            library from the shape);
 *   path     GTR_PATH_AUTO, GTR_PATH_FUSED or GTR_PATH_SPLIT.
 * Any segment length and path give the same result up to rounding; the same
 * shape, segment length and path give bitwise the same result on every call.
 * GTR_PATH_FUSED keeps a 16,640-byte slot per segment and 64-wide key block
 * of a sequence and refuses (GTR_ERR_INVALID_ARG) shapes whose slots exceed
 * 2^31 bytes per sequence (more than 129055 segments at d_k <= 64, 64527
 * above); with d_k > 64 and fp32 I/O its segments hold at most 2 chunks.
 * The initial state makes a long scan splittable: running the two halves of
 * a sequence with the first half's s_final as the second half's s0 equals one
 * call on the whole sequence.
 */
int gtr_gla_fwd_ex(const void *q, const void *k, const void *v, const void *log_gate,
                   void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                   int direction, int dtype, const float *s0, float *s_final,
                   int chunks_per_segment, int path, hipStream_t stream);

/*
 * Runs every check gtr_gla_fwd_ex would run on these arguments (sizes,
 * alignment, overlap, device presence, and that each pointer is device memory
 * of the current device with room for its tensor) and returns the code the
 * call would return before launching anything.  Launches nothing.
 */
int gtr_gla_check(const void *q, const void *k, const void *v, const void *log_gate,
                  void *out, int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                  int direction, int dtype, const float *s0, float *s_final,
                  int chunks_per_segment, int path);

/*
 * Device memory the library keeps for a call of this shape, in bytes: the
 * per-(device, stream) workspace of boundary states and synchronisation
 * words that gtr_gla_fwd (and the typed entry points) would use.  The state
 * itself does not grow with the token count, but intermediate working memory
 * of the scan still does (x-techcon article on GTR, section 架构 /
 * Architecture, on memory beyond the fixed-size state).  Arguments as for
 * gtr_gla_fwd.  Returns 0 on invalid arguments and for calls that need no
 * workspace.  Host-only: touches no device.
 */
size_t gtr_gla_workspace_bytes(int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                               int dtype);

/* The same for a call of gtr_gla_fwd_ex with this segment length and path. */
size_t gtr_gla_workspace_bytes_ex(int B, int H, int grid_h, int grid_w, int d_k, int d_v,
                                  int dtype, int chunks_per_segment, int path);

/* The plan the library uses for a shape: chunks per segment, segments per
 * sequence, and 1 if one fused kernel runs (0: three kernels).  The kernels
 * walk B*H*ceil(d_v/64) sequences, one per 64-wide block of value columns.
 * The plan is that of 16-bit I/O.  fp32 I/O can differ: its one-launch path
 * runs one workgroup per CU instead of two, which moves the automatic choice
 * for some shapes, and with d_k > 64 holds at most 2 chunks per segment.
 * Any output pointer may be NULL.  Returns 0 or an argument error. */
int gtr_gla_plan(int B, int H, int grid_h, int grid_w, int d_k, int d_v, int chunks_per_segment,
                 int path, int *seg_len, int *n_seg, int *fused);

/* Backward pass of gtr_gla_fwd_ex: given dout = dL/dout (laid out like out)
 * and optionally ds_final = dL/ds_final (float32 [B][H][d_k][d_v], NULL = 0),
 * writes dq, dk, dlog_gate (like q) and dv (like v), and ds0 = dL/ds0 when
 * ds0 is not NULL.  s0 is the forward call's initial state (NULL = zero).
 * Gradients follow the recurrence of gtr_gla_fwd by the chain rule (x-techcon
 * article on GTR, section 架构 / Architecture, for the recurrence).  Head dims
 * are multiples of 4 up to 128 (GTR_ERR_UNSUPPORTED otherwise; above 64 key
 * dims, dq, dk, dlog_gate and ds0 are formed one 64-wide key block at a time,
 * since the gate is diagonal; above 64 value dims, dq and dk are summed over
 * the 64-wide value blocks in fp32 before one rounding); every output
 * must be distinct from every input and from the others; the other rules are
 * those of gtr_gla_fwd_ex.  Asynchronous on `stream`; the library keeps a
 * separate per-(device, stream) backward workspace.  The passes along the
 * reversed scan run on a second stream of the library's, forked from `stream`
 * with an event and joined back into it within the call, so the call is
 * ordered on `stream` like a single kernel.  That second stream is made by the
 * first call on a (device, stream): a stream must see one call before it is
 * captured into a graph (GTR_ERR_CAPTURE otherwise).  For 16-bit I/O the
 * states and dq, dk come from fp32 operands; dv comes from the forward
 * kernels run along the reversed scan (keys q, values dout, states dL/dS), so
 * the value-range rules above apply to q, dout and the state gradients. */
int gtr_gla_bwd(const void *q, const void *k, const void *v, const void *log_gate, const void *dout,
                const float *s0, const float *ds_final, void *dq, void *dk, void *dv, void *dlog_gate,
                float *ds0, int B, int H, int grid_h, int grid_w, int d_k, int d_v, int direction,
                int dtype, hipStream_t stream);

/* Message for the last error returned on this thread ("" if none).  The string
 * is owned by the library and stays valid until the next call on this thread. */
const char *gtr_gla_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int gtr_gla_version(void);

/* Frees every cached workspace of this library, forward, backward and Spatial
 * SwiGLU, including the buffers that grown workspaces replaced.  It first
 * synchronises each device that has one.  Graphs captured before this call
 * must not be replayed after it, and no other call of this library may run on
 * another host thread while it does (the calls themselves are thread-safe
 * among each other). */
void gtr_gla_release_workspaces(void);

/*
 * Health of the one-launch path on `stream` (current device).  Its workgroups
 * wait on each other with bounded spins; a wait that gives up (after seconds:
 * only possible if workgroups of the call could not all make progress) leaves
 * that call's outputs undefined and marks the stream's workspace.  This call
 * synchronises `stream`, returns GTR_ERR_TIMEOUT if any wait on it gave up
 * since the previous check (and clears the mark), else GTR_OK.  Not allowed
 * while `stream` is being captured (GTR_ERR_CAPTURE).
 */
int gtr_gla_stream_status(hipStream_t stream);

/*
 * Per-kernel timing (measurement aid).  Between gtr_gla_profile_begin() and
 * gtr_gla_profile_end() every kernel the library launches outside graph
 * capture is bracketed by two HIP events recorded on the stream it runs on
 * (the call's stream, or the backward pass's second stream).  Kernels that
 * run side by side on two streams each count their whole duration.
 * gtr_gla_profile_end() waits for those events and fills, for kernel ids
 * 0..max_kernels-1, the summed elapsed milliseconds and the launch counts
 * (either array may be NULL).  Returns the number of kernel ids (10), or
 * GTR_ERR_LAUNCH if an event could not be read.  Kernel ids: 0 gla_seg_state
 * (segment state contributions), 1 gla_seg_scan (boundary-state scan),
 * 2 gla_seg_out (outputs), 3 gla_fused (the one-kernel path),
 * 4 swiglu_gemm_in, 5 swiglu_mix, 6 swiglu_gemm_out (Spatial SwiGLU),
 * 7 gla_bwd_dqk, 8 gla_bwd_dgate, 9 gla_bwd_ds0 (backward);
 * gtr_gla_kernel_name() returns those names.  The events are taken by the
 * dispatch itself, so they measure kernel execution, not launch overhead.
 */
void gtr_gla_profile_begin(void);
int gtr_gla_profile_end(double *total_ms, int *launches, int max_kernels);
const char *gtr_gla_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* GTR_GLA_H */
