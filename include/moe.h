/*
 * moe.h: C ABI of the routed-expert FFN (qwen3_5-MoE shaped) with low-bit
 * affine expert weights, for one AMD MI355X (gfx950).
 *
 * The layer computed (sources named per entry point below):
 *   logits l[r,e] = W_router[e,:] . x[r,:]  (+ bias[e]),   fp32
 *   gate logit c[r] = w_gate[:] . x[r,:],                    fp32
 *   ids[r,0..k)  = top-k of l[r,:], NaN > +inf > finite, ties to the lower id
 *   p[r,j]       = exp(l[r,ids_j] - l[r,ids_0]) / sum_j' exp(l[r,ids_j'] - l[r,ids_0])
 *   sigma[r]     = 1 / (1 + exp(-c[r]))
 *   per slot j (k routed experts, then the shared expert):
 *     g = Wg x, u = Wu x, h = silu(g) * u, e_j = Wd h
 *   y[r,:]       = sum_j p[r,j] e_j + sigma[r] e_shared      (fp32, slots in pick order)
 * with every weight matrix stored quantised: affine w = s*q + b per group of
 * 64 (MLX-style, 2/3/4/5/6/8-bit), or symmetric w = s*(u-8) per group of 128 (W4A16).
 *
 * Conventions for every call:
 *   - Pointers named dev_* or documented as device memory must point to
 *     device memory of the current HIP device; host_* pointers to host memory.
 *   - All device memory is owned by the caller. The library makes no device
 *     allocation and keeps no global state, except the fixed device array
 *     of moe_forward_windows_noalloc (part of the loaded code object) and
 *     its per-device address; the other calls are reentrant.
 *   - Arguments are validated before anything is enqueued; on an error code
 *     nothing has been enqueued. moe_last_error() (thread-local) then names
 *     the argument, tensor class or format that was refused.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     legacy default stream). Faults inside kernels surface at the caller's
 *     next synchronisation.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null pointer, bad count */
  MOE_EUNSUPPORTED = -2,  /* a format / shape the kernels do not read (refused by name) */
  MOE_ESHAPE = -3,        /* inconsistent shapes */
  MOE_ENOSPACE = -4,      /* destination or workspace too small */
  MOE_EHIP = -5           /* a HIP runtime call failed; moe_last_error() has the hipError_t */
};

/* ----------------------------------------------------------------- formats */
enum moe_mode { MOE_AFFINE = 0, MOE_SYMMETRIC = 1, MOE_DENSE = 2, MOE_MXFP4 = 3 };
enum moe_dtype { MOE_BF16 = 0, MOE_FP16 = 1, MOE_E8M0 = 2 };

/* Quantised format of one tensor class.
 * Accepted combinations (anything else is MOE_EUNSUPPORTED):
 *   {4, 64, MOE_AFFINE, MOE_BF16}     MLX affine 4-bit, group 64
 *       ("Sage-A1.5 ... on the XPU backend #1329", Proposal: affine 4/64 export)
 *   {3, 64, MOE_AFFINE, MOE_BF16}     MLX affine 3-bit, group 64 (routed/shared only)
 *       ("qwen3_5_moe on native CUDA with 3-bit routed experts #803", What I want to run)
 *   {8, 64, MOE_AFFINE, MOE_BF16}     MLX affine 8-bit, group 64 (router, gate row, experts)
 *       (same page and section: routers and the shared-expert gate at 8 bits)
 *   {2, 64, MOE_AFFINE, MOE_BF16}     MLX affine 2-bit, group 64
 *   {5, 64, MOE_AFFINE, MOE_BF16}     MLX affine 5-bit, group 64
 *   {6, 64, MOE_AFFINE, MOE_BF16}     MLX affine 6-bit, group 64
 *                                     (these three: routed/shared only; 5/6-bit experts
 *                                     pair with a shared expert of the same width or 4-bit
 *                                     affine, other pairings are MOE_EUNSUPPORTED)
 *       moe_experts_grouped reads the 3- and 4-bit expert formats in any pairing and
 *       the 2-, 5-, 6- and 8-bit ones with a shared expert of the same width or 4-bit
 *       affine; it refuses the other pairings the decode path reads
 *       (MOE_EUNSUPPORTED, naming the pair; moe_forward_windows reads them)
 *       ("qwen3_5_moe on native CUDA with 3-bit routed experts #803", What exists on
 *       native: the loader reads MLX affine at 2 to 8 bits; Proposal and questions:
 *       affine experts at other widths)
 *   {4, 128, MOE_SYMMETRIC, MOE_FP16} int4 symmetric, group 128, fp16 scales (W4A16)
 *       ("Sage-1.5-W4A16" model card, Model details)
 *   {16, 0, MOE_DENSE, MOE_BF16}      bf16 values (gate row only; the W4A16 export
 *       keeps the shared-expert gate in BF16: same card, Recipe)
 *   {4, 32, MOE_MXFP4, MOE_E8M0}      MXFP4 (routed/shared only): FP4 E2M1 elements in
 *       blocks of 32 sharing one E8M0 exponent byte e, w = e2m1 * 2^(e - 127), e = 255
 *       NaN, no bias (the public OCP Microscaling v1.0 definition: the pages name an
 *       MXFP4-expert checkpoint, "Sage-1.5-W4A16" model card, Performance, decode speed
 *       table, and do not define it). Routed MXFP4 experts pair with an MXFP4 or 4-bit
 *       affine shared expert; read by the decode path, moe_forward_windows and
 *       moe_forward_exact, and by moe_experts_grouped when the layer carries
 *       MOE_LAYER_MX_FP16 (block exponents 104..140 or 255; MOE_EUNSUPPORTED otherwise). */
typedef struct moe_qformat {
  int32_t bits;
  int32_t group;
  int32_t mode;         /* enum moe_mode */
  int32_t scale_dtype;  /* enum moe_dtype: dtype of scales and biases (of values for DENSE) */
} moe_qformat;

/* Shapes and formats of one MoE layer.
 * Supported: hidden % 256 == 0 (<= 4096), n_experts % 64 == 0 (<= 256),
 * 1 <= top_k <= 8, inter and shared_inter % 256 == 0 (<= 2048);
 * act_dtype BF16 or FP16 (the activations x). */
typedef struct moe_layer_desc {
  int32_t hidden, n_experts, top_k, inter, shared_inter, act_dtype;
  moe_qformat router, gate_row, routed, shared;
} moe_layer_desc;

/* One quantised tensor in the canonical (MLX-style) host layout:
 *   codes : uint32 [rows, cols*bits/32]: each row an LSB-first bitstream
 *           (element i in stream bits [bits*i, bits*i+bits), stream bit t is
 *           bit t%32 of word t/32). SYMMETRIC stores the nibble u = q + 8.
 *           DENSE: uint16 bf16 values [rows, cols].
 *   scales: uint16 bit patterns [rows, cols/group] (bf16 or fp16); for E8M0
 *           uint8 exponent bytes [rows, cols/32]
 *   biases: uint16 bit patterns [rows, cols/group] (AFFINE only, else NULL)
 * Stacked routed experts carry a leading [n_experts] axis, experts contiguous. */
typedef struct moe_qtensor {
  const void* codes;
  const void* scales;     /* uint16 entries, or uint8 for E8M0 */
  const uint16_t* biases;
} moe_qtensor;

/* Host sources of one layer (canonical layout, all host memory).
 *   router  [E, H]     gate_row [1, H]
 *   gate, up [E, I, H] down [E, H, I]
 *   sh_gate, sh_up [Is, H]  sh_down [H, Is] */
typedef struct moe_layer_src {
  moe_qtensor router, gate_row, gate, up, down, sh_gate, sh_up, sh_down;
} moe_layer_src;

/* Byte offsets of one packed matrix class inside a packed expert block. */
typedef struct moe_mat_off {
  uint64_t codes, scales;
} moe_mat_off;

/* A packed layer: plain data, owns nothing; valid while `dev` lives.
 * Filled by moe_pack_layer / moe_pack_layer_host; treat as opaque. */
typedef struct moe_layer {
  moe_layer_desc d;
  const void* dev;            /* device base of the packed bytes (NULL until bound) */
  uint64_t bytes;             /* packed size */
  uint64_t router_off, router_scale_off, gate_row_off, gate_row_scale_off;
  uint64_t experts_off, expert_stride;     /* routed expert e at experts_off + e*stride */
  moe_mat_off gu, dn;                      /* inside a routed expert block */
  uint64_t shared_off;
  moe_mat_off sh_gu, sh_dn;                /* inside the shared expert block */
  uint32_t flags;                          /* MOE_LAYER_* bits, set by moe_pack_layer_host */
} moe_layer;

/* moe_layer.flags: MOE_LAYER_MX_FP16 = every E8M0 block exponent of the
 * layer's MXFP4 experts (routed and shared) lies in 104..140 or is 255, so
 * each element times its block scale is exact in fp16 (the grouped GEMMs'
 * operand type); moe_experts_grouped reads MXFP4 experts only then. */
enum moe_layer_flags { MOE_LAYER_MX_FP16 = 1 };

/* Optional per-projection dumps (device memory, fp32), for tests and
 * accuracy reports; any member may be NULL. Layouts use slot index
 * j in [0, k] where j == k is the shared expert:
 *   logits [rows, E+1]   (column E holds the shared-gate logit c)
 *   gu     [rows, k+1, 2, Imax]  (g then u; Imax = max(inter, shared_inter))
 *   h      [rows, k+1, Imax]
 *   e      [rows, k+1, H]        (unweighted slot outputs) */
typedef struct moe_taps {
  float* logits;
  float* gu;
  float* h;
  float* e;
  /* Optional timing: kernel_events[2i] / [2i+1] (hipEvent_t, may be NULL)
   * take the start / end time of the i-th kernel's own dispatch (the kernel
   * is launched with hipExtLaunchKernel), so hipEventElapsedTime gives the
   * kernel's execution time. Kernels: route: 1; decode: gate/up, then
   * down + combine; grouped: sort, gate/up GEMMs, down GEMMs, combine (a
   * phase of two launches takes the first one's start and the second one's
   * end). Events are used only outside stream capture. */
  void* kernel_events[8];
  /* Test hook for the failure path of the decode router (up to 32 rows):
   * 0 (or any positive value) keeps the kernel's own bound on its wait for
   * the tiles' hand-off; a negative value makes the wait end at once, so
   * every row is reported as not handed off (ids -1, NaN p and shared_gate)
   * and the failure is recorded in the workspace (see moe_route_failures). */
  int32_t route_wait_limit;
} moe_taps;

/* ------------------------------------------------------------ pack loader */

/* Packed size in bytes of a layer with descriptor *d.
 * Errors: MOE_EINVAL (null), MOE_EUNSUPPORTED (format/shape refused by name). */
int moe_pack_size(const moe_layer_desc* d, uint64_t* bytes);

/* Repack a layer from the canonical host layout into the kernel layout, into
 * host memory host_dst[0, dst_bytes), and fill *out (out->dev = NULL).
 * Pure host work (no HIP call). The kernel layout: each matrix is cut into
 * tiles of 64 output rows (gate/up tiles hold 32 gate rows then the 32 up
 * rows of the same intermediate indices: gate and up interleaved per tile);
 * codes of a tile are stored chunk-major (32 codes per row per chunk, rows
 * contiguous within a chunk) with each chunk's bits rearranged into 16-bit
 * pairs of consecutive codes; per-group scale/bias words follow per tile.
 * Errors: MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOSPACE (dst_bytes too small). */
int moe_pack_layer_host(const moe_layer_desc* d, const moe_layer_src* src,
                        void* host_dst, uint64_t dst_bytes, moe_layer* out);

/* Set the device base of a layer whose packed bytes the caller has copied
 * to device memory dev_ptr (moe_pack_size bytes, 256-byte aligned). */
int moe_layer_bind(moe_layer* layer, const void* dev_ptr);

/* moe_pack_layer_host into a temporary host buffer, then a synchronous copy
 * to device memory dev_dst (caller-owned, >= moe_pack_size bytes, 256-byte
 * aligned) on `stream`, then moe_layer_bind. Returns when the copy is done.
 * Errors: as moe_pack_layer_host, plus MOE_EHIP. */
int moe_pack_layer(const moe_layer_desc* d, const moe_layer_src* src,
                   void* dev_dst, uint64_t dst_bytes, void* stream, moe_layer* out);

/* Workspace kinds of moe_workspace_size. */
enum moe_ws_kind { MOE_WS_DECODE = 0, MOE_WS_GROUPED = 1, MOE_WS_EXACT = 2 };

/* Workspace bytes for moe_route plus moe_experts_decode (grouped =
 * MOE_WS_DECODE, rows <= 16), plus moe_experts_grouped (MOE_WS_GROUPED), or
 * for moe_forward_exact (MOE_WS_EXACT) at `rows` rows. One buffer of this
 * size serves both calls of a layer (calls on one stream run in order).
 * A workspace must be zero-filled once, before its first use: its first
 * bytes hold the decode router's hand-off words, tagged with a call counter
 * kept beside them, and a sticky failure count (moe_route_failures). Every
 * call leaves them consistent for the next, so the workspace needs no
 * clearing between calls, also when calls are captured and replayed. Any
 * call may use a workspace larger than it needs (say one sized for the most
 * rows of the grouped form); each call checks ws_bytes against its own need
 * (MOE_ENOSPACE). Calls that overlap on one workspace (e.g. on two streams)
 * race; give each stream its own workspace. */
int moe_workspace_size(const moe_layer_desc* d, int rows, int grouped, uint64_t* bytes);

/* ------------------------------------------------------------- hot path */

/* Router of the layer. Source: "qwen3_5_moe on native CUDA with 3-bit routed
 * experts #803", Activity, the "Progress on the 4-bit gate" comment, which
 * gives the routing arithmetic: fp32 logits for every expert and for the
 * shared expert's gate row, the k largest logits picked with equal logits
 * going to the smaller expert id, each pick weighted by the exponential of
 * its logit minus the largest one, and the shared expert added as one more
 * slot scaled by the sigmoid of its gate logit. Here the k weights are also
 * divided by their sum (a reading of that comment).
 *   x          device, [rows, H] activations (act_dtype), row-major
 *   rows       >= 1
 *   logit_bias device, [E] fp32 added to the logits before the pick, or NULL
 *   ids        device, [rows, k] int32, in pick order (logit desc, id asc)
 *   p          device, [rows, k] fp32
 *   shared_gate device, [rows] fp32 sigma(c)
 *   ws         device workspace, >= moe_workspace_size bytes for `rows`,
 *              zero-filled before its first use (see moe_workspace_size)
 *   taps       NULL, or taps->logits / kernel_events (route: 1 kernel)
 * A row holding NaN gets the NaN-ordered picks 0..k-1 and NaN weights.
 * Up to 32 rows run as one launch whose workgroups hand their tiles' picks to
 * one another and must all be resident at once; if another kernel holds the
 * GPU so long that a row's hand-off does not arrive within the kernel's
 * bounded wait, that row gets ids -1 and NaN p and shared_gate (never a pick
 * from missing or stale entries) and the failure is counted in the
 * workspace. The count is sticky: until moe_route_failures clears it, every
 * later call of this router on that workspace reports its rows the same way
 * (so a sequence of calls, such as moe_forward_windows, stops producing
 * results after the first failure instead of continuing silently). */
int moe_route(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
              int32_t* ids, float* p, float* shared_gate, void* ws, uint64_t ws_bytes,
              const moe_taps* taps, void* stream);

/* Routed + shared experts and the combine for decode rows (one row per
 * stream; the per-row form with fp32 sums of the same comment). Expert-centric:
 * rows that picked the same expert share its weight reads, and each row's
 * arithmetic is fixed, so a row's y is bit-identical alone or in a batch.
 *   x       device [rows, H]; rows in 1..16
 *   ids, p, shared_gate  from moe_route on the same layer and x
 *   y       device [rows, H] fp32
 *   ws      device workspace of moe_workspace_size(grouped=0) bytes
 * Preconditions: ids valid for the layer (rows picking an id outside
 * [0, E) get no contribution for that slot); |h| < 65504 (the SwiGLU
 * output enters the down projection as fp16 high + low parts);
 * fp16 activations are used as they are, bf16 ones exactly. */
int moe_experts_decode(const moe_layer* layer, const void* x, int rows, const int32_t* ids,
                       const float* p, const float* shared_gate, float* y, void* ws,
                       uint64_t ws_bytes, const moe_taps* taps, void* stream);

/* Route and experts of any number of rows through the decode step's
 * arithmetic, in consecutive windows of up to 16 rows on `stream`: every
 * row's ids, p, shared_gate and y are bit-identical to its one-row
 * moe_route + moe_experts_decode step, however the rows are cut into calls.
 * Sources: "Native server: --backend xpu for Nemotron on Intel Arc", the
 * review thread (prompt rows and verify windows are to reproduce the one-row
 * step exactly, whatever the cut of the prompt); "Sage-A1.5 ... #1329",
 * Limits to agree on (the grouped form adds in another order than one
 * stream alone). Slower than moe_experts_grouped for wide prompts: each
 * window reads the experts its rows picked. A router failure in one window
 * leaves that window's rows and every later one marked as failed (ids -1,
 * NaN), see moe_route; moe_route_failures reports it.
 *   x, logit_bias, ids, p, shared_gate, y: as moe_route / moe_experts_decode,
 *   for `rows` rows (1..65536)
 *   ws: >= moe_workspace_size(rows = min(rows, 16), grouped = 0) bytes,
 *       zero-filled before its first use
 * Errors: as the two calls; all checks happen before any window is
 * enqueued. Preconditions as moe_experts_decode. */
int moe_forward_windows(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                        int32_t* ids, float* p, float* shared_gate, float* y, void* ws,
                        uint64_t ws_bytes, void* stream);

/* moe_forward_windows without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a fixed device array
 * inside the library, 512 KiB, one copy per GPU, held until the process
 * ends; its address on each device is resolved once, on the first call with
 * that device current. The call allocates nothing.
 *   layer, x, rows, logit_bias, ids, p, shared_gate, y: as moe_forward_windows.
 * Limit: layers whose 16-row decode workspace (moe_workspace_size with
 * rows = min(rows, 16), grouped = 0) exceeds 512 KiB are refused with
 * MOE_ENOSPACE before anything is enqueued (the qwen3_5-MoE 35B-A3B shapes
 * need 329,216 bytes).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two threads) race and must be serialised by the caller.
 * A router failure (see moe_route) marks only the failing call's rows; it is
 * not carried into later calls.
 * Errors: as moe_forward_windows, plus MOE_ENOSPACE as above and MOE_EHIP if
 * the array's device address cannot be resolved. */
int moe_forward_windows_noalloc(const moe_layer* layer, const void* x, int rows, const float* logit_bias,
                                int32_t* ids, float* p, float* shared_gate, float* y, void* stream);

/* A prompt chunk through the layer with the decode step's arithmetic for
 * every row, at chunk cost: each row's ids, weights, gate and y are bit for
 * bit those of its one-row moe_route + moe_experts_decode step, so the
 * result does not depend on how a prompt is cut into calls ("Native server:
 * --backend xpu for Nemotron on Intel Arc", maintainer comment: wide prompts
 * wait until a prompt wider than 16 rows takes the same sum as one row).
 * The router runs the decode router's per-row logits and pick for all rows;
 * the rows are sorted by expert and cut into blocks of at most 16 rows, and
 * gate/up runs the decode kernel's per-row arithmetic on each block (an
 * expert's weights read once per block, not once per 16-row window as in
 * moe_forward_windows); down and the combine are the decode kernel's, per
 * row. Arguments as moe_forward_windows, with a workspace of
 * moe_workspace_size(MOE_WS_EXACT, rows) bytes (zero-filled once, like every
 * workspace); taps as moe_experts_decode plus logits, kernel_events[0..7]
 * bracketing route, sort, gate/up and down.
 *   rows       1 .. 65536
 * Errors: MOE_EINVAL, MOE_ENOSPACE, MOE_EHIP; MOE_EUNSUPPORTED for a shared
 * expert of more than 32 groups per row (an MXFP4 one wider than 1024). */
int moe_forward_exact(const moe_layer* layer, const void* x, int rows, const float* logit_bias, int32_t* ids,
                      float* p, float* shared_gate, float* y, void* ws, uint64_t ws_bytes, const moe_taps* taps,
                      void* stream);

/* The same layer for prompt chunks (the prefill form): rows are sorted by
 * expert (histogram, prefix scan, scatter; a slot's place inside its
 * expert's run is not fixed and no result depends on it), then grouped GEMMs
 * on 16-bit MFMA compute gate/up + SwiGLU and down, then a fixed-order
 * combine. Equal to the decode form within rounding, not bit for bit
 * ("Sage-A1.5 ... #1329", Limits to agree on: the grouped MoE has a
 * different sum order); deterministic from call to call.
 *   rows >= 1 (<= 65536); other arguments as moe_experts_decode, with the
 *   workspace from moe_workspace_size(grouped=1).
 * Preconditions: |x| < 65504 and |h| < 65504 (fp16 MFMA operands).
 * Errors: as moe_experts_decode; MOE_EUNSUPPORTED (nothing enqueued, the
 * message names the reason) for a routed / shared format pair the grouped
 * GEMMs do not read (see moe_qformat) and for MXFP4 experts of a layer
 * without MOE_LAYER_MX_FP16. */
int moe_experts_grouped(const moe_layer* layer, const void* x, int rows, const int32_t* ids,
                        const float* p, const float* shared_gate, float* y, void* ws,
                        uint64_t ws_bytes, const moe_taps* taps, void* stream);

/* Router failures recorded in workspace ws (moe_workspace_size bytes, on
 * the device): *count = the number of rows the decode router reported as
 * failed (ids -1, NaN weights) since the count was last cleared: rows whose
 * hand-off missed the wait bound, and every row of the later calls while the
 * count was nonzero (0 when every call succeeded). With clear != 0 a nonzero count is reset to zero afterwards,
 * which ends the sticky state described at moe_route. Copies 4 bytes to the
 * host and synchronises `stream` (work enqueued before it has finished);
 * not for use during stream capture.
 * Errors: MOE_EINVAL (null), MOE_ENOSPACE (ws_bytes below the fixed router
 * area), MOE_EHIP. */
int moe_route_failures(void* ws, uint64_t ws_bytes, int clear, uint32_t* count, void* stream);

/* ----------------------------------------------------------- diagnostics */
const char* moe_status_string(int status);
const char* moe_last_error(void);   /* thread-local detail of the last failed call */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
