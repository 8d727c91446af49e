/*
 * bmoe.h — C ABI of libbmoe.so: the ButterflyMoE expert-layer forward and
 * its backward on AMD Instinct MI355X (gfx950).
 *
 * Method (ButterflyMoE: Sub-Linear Ternary Experts via Structured Butterfly
 * Orbits, gist.science technical summary):
 *   §2.1  expert i is W_i = B(phi_i) * W_base * B(theta_i)^T, with one ternary
 *         W_base in {-1,0,+1} shared by all experts and butterfly-structured
 *         rotations B(.) holding O(d log d) angles per expert;
 *   §2.3  inference never forms W_i: the input is rotated by B(theta_i)^T,
 *         multiplied by W_base, then rotated by B(phi_i).
 * The layer output of token t with top-k experts e_tj and gates g_tj is
 *   y_t = sum_j g_tj * alpha * B(phi_{e_tj}) W_base B(theta_{e_tj})^T x_t.
 *
 * Readings the pages leave open (fixed here):
 *   - B(a) = S_{L-1}(a_{L-1}) ... S_0(a_0), L = log2 d. Stage s rotates every
 *     pair (i, i + 2^s) with bit s of i clear; pair index p counts those i in
 *     ascending order. A rotation maps (x_i, x_j) to
 *     (c x_i - s x_j, s x_i + c x_j), c = cos a, s = sin a.
 *   - angles are fp32 [N][L][d/2] (expert, stage, pair), theta on the input
 *     side and phi on the output side;
 *   - one fp32 scale alpha multiplies W_base;
 *   - gates are used as given (no renormalisation).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned. The library allocates nothing on the call path and keeps no
 *     state between calls besides the loaded code object.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *     asynchronously; a call returns before the GPU finishes.
 *   - A non-BMOE_OK return comes from host-side validation, before anything
 *     is enqueued; outputs are then untouched. Errors the GPU detects (an
 *     expert id outside [0, N), a W_base entry outside {-1,0,+1}) are written
 *     to a status word in the workspace and read back by bmoe_sync_status().
 *   - Calls are re-entrant for distinct workspaces; two calls sharing one
 *     workspace must be ordered on one stream.
 */
#ifndef BMOE_H
#define BMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BMOE_OK = 0,
  BMOE_E_NULL = 1,       /* a required pointer is NULL */
  BMOE_E_SHAPE = 2,      /* d not a power of two in [2, 8192] (bmoe_forward,
                            bmoe_pack_ternary and the size helpers) or in
                            [16, 8192] (every other entry point; the backward
                            also needs d <= 4096), N < 1 or N > 4096, k < 1 or
                            k > N, T < 0, or T*k beyond 2^31 - 1 */
  BMOE_E_DTYPE = 3,      /* unknown bmoe_dtype */
  BMOE_E_TERNARY = 4,    /* device: a W_base entry outside {-1, 0, +1} */
  BMOE_E_EXPERT = 5,     /* device: an expert id outside [0, N) */
  BMOE_E_WORKSPACE = 6,  /* workspace NULL or smaller than required */
  BMOE_E_HIP = 7,        /* a HIP runtime call failed */
  BMOE_E_ALIGN = 8       /* a pointer is not 16-byte aligned */
} bmoe_status;

/* Storage of the shared substrate: 2-bit words (bmoe_pack_ternary) or the
 * base-3 stream (bmoe_pack_ternary_b3). */
typedef enum { BMOE_W_2BIT = 0, BMOE_W_BASE3 = 1 } bmoe_wformat;

typedef enum {
  BMOE_F32 = 0,   /* x and y fp32; all arithmetic fp32 (substrate product exact
                     to fp32 via a three-way bf16 split of the activations) */
  BMOE_BF16 = 1   /* x and y bf16; rotations in fp32, substrate product on bf16
                     MFMA with fp32 accumulation */
} bmoe_dtype;

/* Number of uint32 words of the packed substrate: d * ceil(d/16). */
size_t bmoe_packed_words(int d);

/* Stored parameters of one layer, d*d + 2 * N * log2(d) * (d/2)
 * (the memory model O(d^2 + N d log d) of §2.2 made exact by the stage layout
 * above). Returns 0 for an invalid d or N. */
size_t bmoe_param_count(int d, int n_experts);

/* Workspace bytes bmoe_forward needs for this shape (0 if the shape is
 * invalid). The workspace holds the routing tables, the per-call rotation
 * coefficient tables (on the shapes that compute them in a separate launch)
 * and the intermediate activations. */
size_t bmoe_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k);

/* Workspace bytes bmoe_pack_ternary needs (a status word). */
size_t bmoe_pack_workspace_bytes(void);

/*
 * Pack the shared ternary substrate (§2.1: entries in {-1,0,+1}) into 2 bits
 * per entry.
 *   w        int8 [d][d], row o = output, column c = input.
 *   packed   uint32 [d][ceil(d/16)] (output). Row o, word g holds columns
 *            c = 16g .. 16g+15 as 2-bit codes, nonzero flag in the low bit
 *            and sign in the high bit (+1 = 01, -1 = 11, 0 = 00): column
 *            v = c - 16g with v = 2j uses bits 2j and 2j+1, v = 2j+1 uses
 *            bits 16+2j and 17+2j.
 *   ws       at least bmoe_pack_workspace_bytes(); receives the status word.
 * Invalid entries are packed as 0 and reported as BMOE_E_TERNARY by
 * bmoe_sync_status(ws, stream).
 */
bmoe_status bmoe_pack_ternary(const int8_t* w, int d, uint32_t* packed, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Base-3 storage of the substrate: the summary (§2.1) stores W_base at 1.58
 * bits per weight (log2 3); this is the byte-aligned form, five ternary
 * digits per byte, 1.6 bits per weight. The d*d entries are taken row-major
 * (entry n = o*d + c); byte j = sum over i < 5 of (w[5j+i] + 1) * 3^i, entry
 * 5j being the least significant digit; digits past d*d are 1 (the value 0).
 * bmoe_packed3_bytes(d) = ceil(d*d / 5) (0 for an invalid d).
 *
 * bmoe_pack_ternary_b3: int8 w [d][d] -> packed3. Invalid entries are stored
 * as 0 and reported as BMOE_E_TERNARY by bmoe_sync_status(ws, stream).
 * bmoe_unpack_ternary_b3: packed3 -> the 2-bit words of bmoe_pack_ternary
 * (bit-identical to packing the same w directly), which bmoe_forward and
 * bmoe_backward take. A byte above 242 is decoded as zeros and reported as
 * BMOE_E_TERNARY. Decoding is one pass that reads d*d/5 bytes and writes
 * d*d/4: it runs once per weight set, or before each forward into a small
 * buffer, rather than inside the product's inner loop.
 * ws: at least bmoe_pack_workspace_bytes() (the status word). The _timed
 * variant records events[0] / events[1] around the decoding kernel.
 */
size_t bmoe_packed3_bytes(int d);
bmoe_status bmoe_pack_ternary_b3(const int8_t* w, int d, uint8_t* packed3, void* ws,
                                 size_t ws_bytes, void* stream);
bmoe_status bmoe_unpack_ternary_b3(const uint8_t* packed3, int d, uint32_t* packed, void* ws,
                                   size_t ws_bytes, void* stream);
bmoe_status bmoe_unpack_ternary_b3_timed(const uint8_t* packed3, int d, uint32_t* packed,
                                         void* ws, size_t ws_bytes, void* stream,
                                         void* const* events);

/*
 * Forward of one ButterflyMoE expert layer for T tokens (§2.3 order).
 *   dt        BMOE_F32 or BMOE_BF16: element type of x and y.
 *   x         [T][d] tokens.
 *   ids       int32 [T][k] expert ids in [0, N). Routed index r = t*k + j.
 *   gates     fp32 [T][k] gate weights g_tj.
 *   theta     fp32 [N][log2 d][d/2] input-side angles.
 *   phi       fp32 [N][log2 d][d/2] output-side angles.
 *   w_packed  uint32 [d][ceil(d/16)] from bmoe_pack_ternary.
 *   alpha     scale of W_base.
 *   y         [T][d] output (must not alias x).
 *   ws        workspace of at least bmoe_workspace_bytes(dt, T, d, N, k).
 *   route_out optional (may be NULL): int32 [N+1 + 2*T*k] receiving
 *             offsets[N+1] (exclusive prefix of per-expert row counts),
 *             perm[T*k] (sorted slot -> routed index; experts ascending,
 *             ascending r within an expert) and inv[T*k] (routed index ->
 *             sorted slot). These are the tables the forward itself uses.
 * T = 0 is a no-op. Bad expert ids are clamped for addressing (so every
 * access stays in bounds) and reported by bmoe_sync_status(); y is then
 * unspecified.
 * d is a power of two from 2 to 8192. For d = 2, 4 or 8 one thread per token
 * runs its k rows after the preparation launch: Z is rounded to the
 * activation type before the product, H stays fp32, and each gate-weighted
 * row is rounded to the activation type before the fp32 sum over j.
 * For bf16 with d = 256 or 512 one kernel does the whole per-row
 * computation (then the combine): with T*k <= 8192 and N <= 256 (N <= 512
 * at d = 256) it routes its rows itself, otherwise it follows a preparation
 * launch that only
 * routes. It evaluates the rotation coefficients on the hardware sine/cosine
 * unit (at most 4e-7 absolute error for angles up to 1000 in magnitude).
 * Other shapes compute them with sincosf in a preparation launch. Both are
 * far inside the bf16 tolerance, but the two are not bit-identical.
 */
bmoe_status bmoe_forward(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                         const int32_t* ids, const float* gates, const float* theta,
                         const float* phi, const uint32_t* w_packed, float alpha, void* y,
                         void* ws, size_t ws_bytes, int32_t* route_out, void* stream);

/* Number of kernels bmoe_forward enqueues for this shape (0 if invalid), and
 * the name of kernel i (as it appears in a kernel trace). */
int bmoe_forward_kernel_count(bmoe_dtype dt, int T, int d, int n_experts, int k);
const char* bmoe_forward_kernel_name(bmoe_dtype dt, int T, int d, int n_experts, int k, int i);

/*
 * bmoe_forward, additionally timing each kernel's own dispatch: kernel i is
 * launched with events[2i] as its start event and events[2i+1] as its stop
 * event (hipExtLaunchKernel), so hipEventElapsedTime(events[2i],
 * events[2i+1]) is that kernel's execution time, without launch gaps.
 * `events` holds 2 * bmoe_forward_kernel_count(...) hipEvent_t created by the
 * caller on the current device (NULL behaves as bmoe_forward). Results are
 * identical to bmoe_forward.
 */
bmoe_status bmoe_forward_timed(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                               const int32_t* ids, const float* gates, const float* theta,
                               const float* phi, const uint32_t* w_packed, float alpha, void* y,
                               void* ws, size_t ws_bytes, int32_t* route_out, void* stream,
                               void* const* events);

/*
 * The shared-substrate product alone (§2.3, the middle step): for bf16 Z
 * [M][d] (row-major; rows are routed rows after the input-side rotation),
 * H [M][d] = alpha * Z * W_base^T in bf16, with fp32 accumulation over K in
 * ascending 16-wide slices on bf16 MFMA (exact ternary products).
 *   w       the substrate in format fmt: BMOE_W_2BIT, uint32 [d][d/16] from
 *           bmoe_pack_ternary; BMOE_W_BASE3, the stream of
 *           bmoe_pack_ternary_b3 (bmoe_packed3_bytes(d) bytes) in a buffer of
 *           at least bmoe_packed3_bytes(d) + 8 bytes (the kernel reads whole
 *           aligned dwords; the bytes past the stream are never decoded), whose
 *           digits the kernel decodes as it stages each K-step of the
 *           substrate (a 256-entry LDS table).
 *   d       a multiple of 128 in [128, 8192]; M >= 0 (0: no-op).
 * Both formats run the same kernel and give bit-identical H. z, w, h: device
 * pointers, 16-byte aligned; h must not alias z. events (may be NULL):
 * events[0] / events[1] become the kernel's start and stop events.
 */
bmoe_status bmoe_product(int M, int d, const void* z, const void* w, bmoe_wformat fmt,
                         float alpha, void* h, void* stream, void* const* events);

/*
 * bmoe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is a fixed array in the library's
 * device memory, BMOE_NOALLOC_MAX_WORKSPACE bytes on each GPU the library
 * runs on, held until the process ends. Nothing is allocated on any call:
 * no hipMalloc, hipFree or allocating library routine.
 *   Arguments as bmoe_forward, without ws / ws_bytes, plus
 *   status  nullable device int32: receives BMOE_OK, or BMOE_E_EXPERT for an
 *           expert id outside [0, N) (read it with bmoe_sync_status(status,
 *           stream)); NULL: such errors are not reported. 4-byte aligned.
 * Returns BMOE_E_WORKSPACE when the shape needs more than
 * BMOE_NOALLOC_MAX_WORKSPACE bytes of workspace (compare
 * bmoe_workspace_bytes(dt, T, d, N, k) with it), before anything is
 * enqueued. Results are identical to bmoe_forward's.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, or other threads
 * without ordering) race and give undefined results; order them on one
 * stream. The array's address is looked up once per GPU, on the first call
 * that runs there (the GPU of `stream`, or the current one for NULL).
 */
#define BMOE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
bmoe_status bmoe_forward_noalloc(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                 const void* x, const int32_t* ids, const float* gates,
                                 const float* theta, const float* phi, const uint32_t* w_packed,
                                 float alpha, void* y, int32_t* route_out, int32_t* status,
                                 void* stream);

/* Wait for `stream`, then return the device-side status of the last call
 * that used `ws` (bmoe_forward, bmoe_backward, bmoe_rotate_in, or a pack or
 * base-3 unpack): BMOE_OK, BMOE_E_EXPERT or BMOE_E_TERNARY, or BMOE_E_HIP if
 * the wait itself failed. */
bmoe_status bmoe_sync_status(const void* ws, void* stream);

/* Workspace bytes bmoe_backward needs for this shape (0 if the shape is not
 * supported: as bmoe_forward, and 16 <= d <= 4096). */
size_t bmoe_backward_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k);

/*
 * Backward of the layer computed by bmoe_forward, for training the rotations
 * (gist.science summary, §2.4; the map itself §2.1/§2.3). Given dy = dL/dy
 * (same dtype and layout as y), writes the gradients of L:
 *   dx      [T][d], dtype dt       sum over j of B(theta_e) dz
 *   dgates  fp32 [T][k]            <dy_t, B(phi_e) h> for routed row (t, j)
 *   dtheta, dphi  fp32 [N][L][d/2] per-stage, per-pair angle gradients
 *                                  (experts without rows get 0)
 *   dw      fp32 [d][d] or NULL    alpha * sum over routed rows of dh z^T:
 *                                  the substrate's gradient taken as a real
 *                                  matrix (the straight-through reading),
 *                                  row o = output, column c = input
 * with z = B(theta_e)^T x_t, h = alpha W_base z, dh = B(phi_e)^T (g dy_t).
 * The other arguments are bmoe_forward's (same routing and rounding points;
 * the forward is recomputed inside). All outputs are overwritten; dtheta and
 * dphi are summed per expert in a fixed order (run-to-run bit-identical). The
 * dw product is a plain GEMM over the routed rows, one launch of the
 * library's own kernel (bf16 MFMA for bf16 with 128 <= d <= 4096, fp32 MFMA
 * otherwise); when d is small it is split into row ranges whose fp32
 * products are summed in a fixed order.
 * ws: at least bmoe_backward_workspace_bytes(), 16-byte aligned. Errors as
 * bmoe_forward.
 */
bmoe_status bmoe_backward(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                          const int32_t* ids, const float* gates, const float* theta,
                          const float* phi, const uint32_t* w_packed, float alpha,
                          const void* dy, void* dx, float* dgates, float* dtheta, float* dphi,
                          float* dw, void* ws, size_t ws_bytes, void* stream);

/* Number and names of the launches of one bmoe_backward (0 / "" when the
 * shape is unsupported or T == 0, or i is out of range). The substrate
 * gradient's slot ("dw_kernel") launches nothing when dw is NULL. */
int bmoe_backward_kernel_count(bmoe_dtype dt, int T, int d, int n_experts, int k);
const char* bmoe_backward_kernel_name(bmoe_dtype dt, int T, int d, int n_experts, int k, int i);

/*
 * bmoe_backward, additionally timing each launch: launch i records
 * events[2i] and events[2i+1] around its own execution, as in
 * bmoe_forward_timed (with dw NULL, the dw_kernel slot's two events are
 * recorded back to back on `stream`). `events` holds 2 * bmoe_backward_kernel_count(...)
 * hipEvent_t created by the caller on the current device; NULL behaves as
 * bmoe_backward. Results are identical to bmoe_backward.
 */
bmoe_status bmoe_backward_timed(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                const void* x, const int32_t* ids, const float* gates,
                                const float* theta, const float* phi, const uint32_t* w_packed,
                                float alpha, const void* dy, void* dx, float* dgates,
                                float* dtheta, float* dphi, float* dw, void* ws, size_t ws_bytes,
                                void* stream, void* const* events);

/*
 * Forward that keeps its intermediates for the backward (a training step):
 * as bmoe_forward, but after the call the workspace holds the routing
 * tables, both cos/sin tables, Z and H (bf16 d = 256, 512: the fused kernel
 * after the preparation launch writes Z and H beside its U rows; other
 * shapes: the unfused path). bmoe_backward_kept then reads them instead of
 * recomputing the forward; bmoe_backward recomputes them with the same
 * kernels, so the gradients of the two are bit-identical. No route_out (the
 * tables stay in the workspace). ws: at least
 * bmoe_forward_keep_workspace_bytes(). y is that of bmoe_forward up to the
 * rounding of the path taken (the same fused or unfused kernels).
 */
size_t bmoe_forward_keep_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k);
bmoe_status bmoe_forward_keep(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                              const int32_t* ids, const float* gates, const float* theta,
                              const float* phi, const uint32_t* w_packed, float alpha, void* y,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * bmoe_backward after a bmoe_forward_keep: fwd_ws (fwd_ws_bytes) is that
 * call's workspace, unchanged since; x, gates, w_packed and alpha are the
 * same as in that call (ids, theta and phi live on in its tables). Skips the
 * forward recompute (routing, cos/sin, Z, H); the results are bit-identical
 * to bmoe_backward's. fwd_ws is only read. ws: at least
 * bmoe_backward_workspace_bytes(). The _timed variant has the same launch
 * slots as bmoe_backward_timed; the slots of the skipped launches are empty.
 */
bmoe_status bmoe_backward_kept(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                               const float* gates, const uint32_t* w_packed, float alpha,
                               const void* dy, void* dx, float* dgates, float* dtheta,
                               float* dphi, float* dw, const void* fwd_ws, size_t fwd_ws_bytes,
                               void* ws, size_t ws_bytes, void* stream);
bmoe_status bmoe_backward_kept_timed(bmoe_dtype dt, int T, int d, int n_experts, int k,
                                     const void* x, const float* gates,
                                     const uint32_t* w_packed, float alpha, const void* dy,
                                     void* dx, float* dgates, float* dtheta, float* dphi,
                                     float* dw, const void* fwd_ws, size_t fwd_ws_bytes, void* ws,
                                     size_t ws_bytes, void* stream, void* const* events);

/*
 * Input-side rotation alone (§2.3, first step): z[r] = B(theta_e)^T x[t] for
 * every routed row r = t*k + j, e = ids[t][j], written in routed order
 * ([T*k][d], dtype dt; the same rounding point as the forward's Z). Used to
 * measure how the rotation spreads activation outliers (§2.4). ws: at least
 * bmoe_rotate_in_workspace_bytes() (routing tables and cos/sin; its status
 * word reports bad expert ids through bmoe_sync_status). Shapes and errors
 * as bmoe_forward.
 */
size_t bmoe_rotate_in_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k);
bmoe_status bmoe_rotate_in(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                           const int32_t* ids, const float* theta, void* z, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Per-row quantisation error of src [rows][d] (dtype dt), for the
 * outlier-spreading measurement (§2.4, §4: the rotation lowers the activation
 * quantisation error; the pages name no quantiser, so this is the plain
 * per-token symmetric one). For row v:
 *   s = max|v| / m (mode 0, absmax; m = 127 for int8, 7 for int4, 1 for
 *       ternary) or s = mean|v| (mode 1, absmean),
 *   q = s * clip(rint(v / s), -m, m),
 *   err[row]   = ||v - q|| / ||v||        (fp32; 0 for a zero row),
 *   crest[row] = max|v| / rms(v)          (fp32; optional, may be NULL).
 * d as bmoe_forward, rows >= 0, m >= 1, mode 0 or 1 (BMOE_E_SHAPE otherwise).
 */
bmoe_status bmoe_quant_error(bmoe_dtype dt, int rows, int d, const void* src, int m, int mode,
                             float* err, float* crest, void* stream);

/*
 * Router: the top-k gate that picks each token's experts and gates (the
 * layer is a top-k mixture of experts, ButterflyMoE abstract and summary
 * §2.3; the pages give no router formula, so this is the plain top-k
 * softmax gate). For token t:
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c]     (fp32 accumulation)
 *   ids[t][0..k)  the k experts with the largest logits, in descending
 *                 order of logit; equal logits go to the lower expert id
 *   gates[t][j]   softmax over the k chosen logits (they sum to 1)
 * The outputs are laid out exactly as bmoe_forward's ids and gates inputs.
 *   dt        element type of x and w_router (bf16: products on bf16 MFMA,
 *             fp32 accumulation; fp32: fp32 FMA).
 *   x         [T][d].
 *   w_router  [N][d]: one row per expert (W_r stored transposed).
 *   ids       int32 [T][k] (output).
 *   gates     fp32 [T][k] (output).
 *   logits    optional fp32 [T][N] output; NULL keeps the logits in ws.
 *   ws        needed only when logits is NULL: at least
 *             bmoe_router_workspace_bytes() bytes.
 * Shapes as bmoe_forward, and k <= 64 (BMOE_E_SHAPE otherwise). Logits that
 * are NaN give unspecified ids.
 */
size_t bmoe_router_workspace_bytes(bmoe_dtype dt, int T, int d, int n_experts, int k);
bmoe_status bmoe_router(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                        const void* w_router, int32_t* ids, float* gates, float* logits,
                        void* ws, size_t ws_bytes, void* stream);

/* bmoe_router, timing its two launches (logits, then top-k): events holds 4
 * hipEvent_t (start/stop of each), or NULL. Results identical to bmoe_router. */
bmoe_status bmoe_router_timed(bmoe_dtype dt, int T, int d, int n_experts, int k, const void* x,
                              const void* w_router, int32_t* ids, float* gates, float* logits,
                              void* ws, size_t ws_bytes, void* stream, void* const* events);

/* Static description of a status code. */
const char* bmoe_status_str(bmoe_status s);

/*
 * Measured ceilings, reported by the benchmark beside the published peaks
 * (they are not part of the layer). Each launches one kernel on `stream`,
 * with events[0] / events[1] (may be NULL) as the start and stop events of
 * its own dispatch.
 *   bmoe_ceiling_mfma_bf16: chains of v_mfma_f32_32x32x16_bf16 on register
 *     operands, eight waves per SIMD on every CU; *flops (may be NULL)
 *     receives the multiply-add flops it executes (iters scales them).
 *   bmoe_ceiling_valu_f32: chains of fp32 fused multiply-adds (no packed
 *     ops), eight waves per SIMD; *flops as above.
 *   sink: device fp32 [BMOE_CEILING_SINK_FLOATS], overwritten.
 *   bmoe_ceiling_copy: a plain copy of `bytes` (a multiple of 16) from src to
 *     dst, both 16-byte aligned device buffers; reads and writes `bytes`.
 */
#define BMOE_CEILING_SINK_FLOATS (256 * 8 * 256)
bmoe_status bmoe_ceiling_mfma_bf16(int iters, float* sink, void* stream, void* const* events,
                                   double* flops);
bmoe_status bmoe_ceiling_valu_f32(int iters, float* sink, void* stream, void* const* events,
                                  double* flops);
bmoe_status bmoe_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream,
                              void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* BMOE_H */
