/*
 * ssd.h -- C ABI of the MI355X (gfx950) complex chunkwise SSD scan library.
 *
 * The operation is the complex-valued selective state-space scan of the
 * Mamba-3-Lite pages. For every batch row b and head h, independently:
 *
 *   Abar_t = exp(softplus(dt_t) * A_h)                       (discretisation)
 *   s_t    = Abar_t * s_{t-1} + B_t (outer) x_t              (state, N x D)
 *   y_t    = Re( sum_n C_t[n] * s_t[n, :] )                   (output, D)
 *
 * with no conjugation anywhere, s_{-1} the initial state (zero by default)
 * and final_state = s_{T-1}. Sources: "Extending -- SSM variants & Triton
 * kernels" (Path A Step 1: the naive scan and the discretisation; Step 3: the
 * chunkwise function returns the real part), "index.html" lab 03 (the
 * chunkwise decomposition: per-chunk log-decay running sums, the masked
 * decay matrix L, the intra-chunk term, per-chunk states and the passing of
 * states between chunks), and "Skills Reference" Skill 3 (chunk_size 32..256,
 * default 64).
 *
 * Gradients (ssd_chunk_backward) follow from the same recurrence by reverse-mode
 * differentiation.
 *
 * Conventions common to every call:
 *   * All tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates no memory and keeps no state between calls.
 *   * Layouts are dense row-major. Complex numbers are interleaved (re, im)
 *     pairs of float32, bit-identical to torch.complex64.
 *   * Argument checks run before anything is launched; a failed check returns
 *     a negative status and touches no memory. Work is launched on `stream`
 *     and is asynchronous; a launch failure returns SSD_ERR_HIP.
 *   * There is one code path: no fallback exists when a check fails.
 *   * Calls on different streams with different workspaces are independent.
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream, or NULL for the null stream. The same type as hipStream_t
 * (a pointer to struct ihipStream_t), declared here so that this header needs
 * no HIP header. */
typedef struct ihipStream_t *ssd_stream_t;

/* One complex64 value, laid out as torch.complex64. */
typedef struct {
    float re, im;
} ssd_c64;

enum {
    SSD_OK = 0,
    SSD_ERR_NULL = -1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = -2,       /* a size is negative, or N, D, chunk_size < 1 */
    SSD_ERR_ODD_N = -3,       /* N is odd: the state must pack into real pairs */
    SSD_ERR_BLOCK_DIMS = -4,  /* N, D or chunk_size above 256 */
    SSD_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
    SSD_ERR_ALIGN = -6,       /* a pointer is not aligned as documented */
    SSD_ERR_HIP = -7,         /* the HIP runtime reported an error */
    SSD_ERR_UNSUPPORTED = -8, /* a valid size this build does not cover yet */
    SSD_ERR_ALIAS = -9        /* an output overlaps an input it must not */
};

/* Largest N, D and chunk_size accepted (the pages cap kernel blocks at 256). */
#define SSD_MAX_BLOCK 256

/*
 * ssd_discretise -- the discretisation step and the per-chunk cumulative
 * log-decay ("Extending", Path A Step 1 and Path B Step 2; index.html lab 03).
 *
 *   dt        (batch, T, H) float32, step logits.
 *   A         (H) complex64, one eigenvalue per head.
 *   A_bar     out, nullable: (batch, T, H) complex64, exp(softplus(dt) * A).
 *   log_decay_cumsum
 *             out, nullable: (batch, H, nc, chunk_size) complex64 with
 *             nc = ceil(T / chunk_size). Entry [b,h,c,l] is the sum of
 *             softplus(dt_t) * A_h over t = c*chunk_size .. c*chunk_size + l.
 *             Positions of a last partial chunk past T repeat the final sum.
 *   chunk_size 0 when log_decay_cumsum is NULL, else 1..256.
 * Alignment: 4 bytes for dt, 8 bytes for the complex arrays.
 * batch, T or H equal to 0 is a no-op.
 */
int ssd_discretise(const float *dt, const ssd_c64 *A, int64_t batch, int64_t T, int64_t H,
                   int64_t chunk_size, ssd_c64 *A_bar, ssd_c64 *log_decay_cumsum,
                   ssd_stream_t stream);

/*
 * ssd_chunk_forward_workspace_bytes -- device workspace that ssd_chunk_forward
 * needs for these sizes (0 when none is needed). The value depends only on
 * the arguments. Negative or invalid sizes return 0.
 */
size_t ssd_chunk_forward_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t N,
                                         int64_t D, int64_t chunk_size);

/*
 * ssd_chunk_forward -- the chunkwise complex SSD scan forward
 * ("Extending", Path A Step 3: the chunkwise function; index.html lab 03).
 *
 *   x            (batch, T, H, D) complex64, token content.
 *   A            (H) complex64.
 *   B_t, C_t     (batch, T, H, N) complex64, input and output maps.
 *   dt           (batch, T, H) float32.
 *   chunk_size   1..256; a last chunk shorter than chunk_size is allowed
 *                (T need not be a multiple of it). It sets the span of the
 *                intra-chunk quadratic term, up to 64 tokens: a longer chunk is
 *                evaluated as 64-token sub-chunks with the state passed between
 *                them. The result does not depend on chunk_size beyond rounding.
 *   initial_state nullable: (batch, H, N, D) complex64 state s_{-1}; NULL
 *                means zero.
 *   y            out: (batch, T, H, D) float32, the real part of the output.
 *   final_state  out, nullable: (batch, H, N, D) complex64, s_{T-1}.
 *   workspace    device scratch of at least
 *                ssd_chunk_forward_workspace_bytes(...) bytes, 256-byte
 *                aligned; may be NULL when that size is 0. Its contents on
 *                entry are ignored. It is needed when there are fewer
 *                (batch, head) sequences than the GPU has compute units (the
 *                sequences are then cut into segments) and when N > 64 (the
 *                state is then split into 64-row slices whose partial outputs
 *                are added up).
 * Constraints: N even (SSD_ERR_ODD_N); N, D, chunk_size <= 256
 * (SSD_ERR_BLOCK_DIMS).
 * Alignment: x, A, B_t, C_t, initial_state, final_state 8 bytes (B_t and C_t
 * rows are read 16 bytes at a time, at any 8-byte alignment); dt and y 4 bytes.
 * batch or H equal to 0 is a no-op; T equal to 0 copies initial_state (or
 * zeros) into final_state.
 */
int ssd_chunk_forward(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t, const ssd_c64 *C_t,
                      const float *dt, int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                      int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                      ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                      ssd_stream_t stream);

/* Size of the static device scratch of ssd_chunk_forward_noalloc (32 MiB per GPU). */
#define SSD_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * ssd_chunk_forward_noalloc -- ssd_chunk_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same scan, with the same arguments minus
 * the workspace. The workspace lives in a static device array of
 * SSD_NOALLOC_SCRATCH_BYTES bytes, one per GPU, created when the library's code
 * object is loaded on that GPU and held until the process ends; this call and
 * the kernels it launches allocate nothing.
 *   Arguments, constraints, alignment and results: as ssd_chunk_forward.
 *   SSD_ERR_WORKSPACE when ssd_chunk_forward_workspace_bytes(...) for these
 *   sizes exceeds SSD_NOALLOC_SCRATCH_BYTES (checked before anything runs).
 * The scratch used is that of the current device; `stream` must belong to it.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (different streams, or host threads) race and must be
 * serialised by the caller. Its contents on entry are ignored.
 */
int ssd_chunk_forward_noalloc(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t,
                              const ssd_c64 *C_t, const float *dt, int64_t batch, int64_t T,
                              int64_t H, int64_t N, int64_t D, int64_t chunk_size,
                              const ssd_c64 *initial_state, float *y, ssd_c64 *final_state,
                              ssd_stream_t stream);

/*
 * ssd_chunk_forward_proj -- the same scan read straight from the in_proj output
 * ("Extending", Path A Step 2: Mamba3Block._forward_impl slices the projection
 * of each token into x (H*D), four H*N blocks and a trailing dt (H); the
 * in_proj width is H*(D + 4N + 1)). x is real here, and B_t, C_t are given by
 * their real and imaginary blocks.
 *
 *   proj         (batch, T, token_stride) float32; the row of token (b, t) is
 *                  [ x (H, D) | Re B_t (H, N) | Im B_t (H, N) |
 *                    Re C_t (H, N) | Im C_t (H, N) | dt (H) | unused ]
 *                (the order of the four N-blocks is this library's reading).
 *   token_stride floats between consecutive token rows, >= H*(D + 4N + 1),
 *                even. Floats past the last block are never read.
 *   A, chunk_size, initial_state, y, final_state, workspace: as for
 *                ssd_chunk_forward; the workspace size is
 *                ssd_chunk_forward_workspace_bytes(batch, T, H, N, D, chunk_size).
 * Result: identical in exact arithmetic to ssd_chunk_forward with
 * x = x_real + 0i, B_t = Re B + i Im B, C_t = Re C + i Im C.
 * Constraints: as ssd_chunk_forward; token_stride <= 2^22 (SSD_ERR_UNSUPPORTED).
 * Alignment: proj 8 bytes and H*D even (the N-blocks are read as float pairs),
 * else SSD_ERR_ALIGN.
 */
int ssd_chunk_forward_proj(const float *proj, int64_t token_stride, const ssd_c64 *A,
                           int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                           int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                           ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                           ssd_stream_t stream);

/*
 * ssd_chunk_forward_proj_bf16 -- ssd_chunk_forward_proj with the in_proj rows
 * in bfloat16 ("AGENTS & System Architecture": the model trains in BF16
 * (section 1, subagent notes) while the recurrent state stays complex64
 * (section 3, numerical-stability rules)). proj holds bfloat16 bit patterns
 * (uint16); each element is
 * widened to float32 as it is loaded and every product, sum and the state
 * stay float32, so the result equals ssd_chunk_forward_proj on the widened
 * rows. Same arguments, constraints and workspace as ssd_chunk_forward_proj,
 * except the alignment: proj 4 bytes (and token_stride, H*D even).
 */
int ssd_chunk_forward_proj_bf16(const uint16_t *proj, int64_t token_stride, const ssd_c64 *A,
                                int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                                int64_t chunk_size, const ssd_c64 *initial_state, float *y,
                                ssd_c64 *final_state, void *workspace, size_t workspace_bytes,
                                ssd_stream_t stream);

/*
 * ssd_chunk_backward_workspace_bytes -- device workspace that
 * ssd_chunk_backward needs for these sizes (0 when T, batch or H is 0, or the
 * sizes are invalid). It holds the state entering and the adjoint leaving
 * every chunk, in 64 x 64 blocks: about 2 * batch * H * ceil(T / min(chunk_size,
 * 32)) * ceil(N/64) * ceil(D/64) * 32 KiB; with N or D above 64 also the
 * per-slice partial gradients (8 * batch * T * H * (ceil(N/64) D +
 * 2 ceil(D/64) N) + 4 * batch * T * H * ceil(N/64) ceil(D/64) bytes).
 */
size_t ssd_chunk_backward_workspace_bytes(int64_t batch, int64_t T, int64_t H, int64_t N,
                                          int64_t D, int64_t chunk_size);

/*
 * ssd_chunk_backward -- gradients of the chunkwise scan ("Extending", Path B
 * Step 3: the backward of a scan's autograd Function is seeded with the true
 * upstream gradients of y and final_state and returns a gradient for every
 * differentiated input).
 *
 * For the loss l = sum(grad_y * y) + sum(Re(conj(grad_final_state) * final_state))
 * of the forward call with the same inputs, each output receives dl/dRe(z) +
 * i dl/dIm(z) for a complex input z (the convention of torch's autograd for
 * complex tensors) and dl/dz for a real one:
 *   x, A, B_t, C_t, dt, initial_state, chunk_size
 *                  as for ssd_chunk_forward (initial_state nullable = zero).
 *   grad_y         (batch, T, H, D) float32, upstream gradient of y.
 *   grad_final_state nullable: (batch, H, N, D) complex64; NULL means zero.
 *   grad_x         out: (batch, T, H, D) complex64.
 *   grad_A         out: (H) complex64, summed over batch rows and time.
 *   grad_B_t, grad_C_t out: (batch, T, H, N) complex64.
 *   grad_dt        out: (batch, T, H) float32.
 *   grad_initial_state out, nullable: (batch, H, N, D) complex64.
 *   workspace      device scratch of at least
 *                  ssd_chunk_backward_workspace_bytes(...) bytes, 256-byte
 *                  aligned (required whenever T > 0). Contents on entry ignored.
 * The chunk evaluated at once is min(chunk_size, 32) tokens; the result does
 * not depend on chunk_size beyond rounding. With N or D above 64 the state is
 * evaluated in 64 x 64 blocks whose partial gradients are added in a fixed
 * order (deterministic).
 * Constraints: as ssd_chunk_forward (N even; N, D, chunk_size <= 256), and
 * batch * H * ceil(N/64) * ceil(D/64) * ceil(T / min(chunk_size, 32)) below 2^31
 * (the chunks are indexed with 32-bit integers; SSD_ERR_UNSUPPORTED otherwise, and
 * the workspace size is then 0).
 * Alignment: complex arrays 8 bytes; dt, grad_y, grad_dt 4 bytes.
 * batch or H equal to 0 is a no-op; T equal to 0 writes grad_final_state (or
 * zeros) to grad_initial_state and zeros to grad_A.
 */
int ssd_chunk_backward(const ssd_c64 *x, const ssd_c64 *A, const ssd_c64 *B_t, const ssd_c64 *C_t,
                       const float *dt, int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                       int64_t chunk_size, const ssd_c64 *initial_state, const float *grad_y,
                       const ssd_c64 *grad_final_state, ssd_c64 *grad_x, ssd_c64 *grad_A,
                       ssd_c64 *grad_B_t, ssd_c64 *grad_C_t, float *grad_dt,
                       ssd_c64 *grad_initial_state, void *workspace, size_t workspace_bytes,
                       ssd_stream_t stream);

/*
 * ssd_chunk_backward_proj -- ssd_chunk_backward for the scan read from in_proj
 * rows (ssd_chunk_forward_proj, float32 rows): the gradients are written as
 * gradient rows of the same layout.
 *   proj, token_stride, A, chunk_size, initial_state, grad_y, grad_final_state,
 *                as for ssd_chunk_forward_proj and ssd_chunk_backward.
 *   grad_proj    out: (batch, T, token_stride) float32; in each token row the x
 *                block receives dl/dx (x is real), the Re/Im B and C blocks the
 *                real and imaginary parts of the B_t and C_t gradients, the dt
 *                block dl/ddt. Floats past the blocks are not written.
 *   grad_A, grad_initial_state, workspace: as for ssd_chunk_backward (same
 *                workspace size).
 * Constraints: as ssd_chunk_backward.
 * Alignment: proj, grad_proj, grad_y 4 bytes; A and the states 8 bytes.
 */
int ssd_chunk_backward_proj(const float *proj, int64_t token_stride, const ssd_c64 *A,
                            int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                            int64_t chunk_size, const ssd_c64 *initial_state, const float *grad_y,
                            const ssd_c64 *grad_final_state, float *grad_proj, ssd_c64 *grad_A,
                            ssd_c64 *grad_initial_state, void *workspace, size_t workspace_bytes,
                            ssd_stream_t stream);

/*
 * ssd_chunk_backward_proj_bf16 -- ssd_chunk_backward_proj for bfloat16 rows (the
 * training precision of AGENTS & System Architecture: BF16 activations, the
 * recurrent state complex64): proj and grad_proj hold bfloat16 values as their
 * 16-bit patterns. Rows are widened to float32 as they are loaded; every
 * product, sum and stored state stays float32 (as in ssd_chunk_forward_proj_bf16),
 * and each gradient is rounded to bfloat16 (nearest, ties to even) as it is
 * stored. grad_y, grad_final_state, grad_A and grad_initial_state stay float32
 * / complex64.
 * Arguments, constraints and workspace: as ssd_chunk_backward_proj.
 * Alignment: proj, grad_proj 2 bytes; grad_y 4 bytes; A and the states 8 bytes.
 */
int ssd_chunk_backward_proj_bf16(const uint16_t *proj, int64_t token_stride, const ssd_c64 *A,
                                 int64_t batch, int64_t T, int64_t H, int64_t N, int64_t D,
                                 int64_t chunk_size, const ssd_c64 *initial_state,
                                 const float *grad_y, const ssd_c64 *grad_final_state,
                                 uint16_t *grad_proj, ssd_c64 *grad_A,
                                 ssd_c64 *grad_initial_state, void *workspace,
                                 size_t workspace_bytes, ssd_stream_t stream);

/*
 * ssd_head_mix -- the MIMO head mixer that follows the scan (index.html lab 02
 * "MIMO MIXER": fully connected across the SSM heads, 1024 -> 1024 as 16 heads
 * of 64 channels, identity at initialisation; "Knows cold" item 2 of the AGENTS
 * page; the in_proj -> scan -> MIMO -> out_proj order of "Extending", Path A;
 * the model's parameter count in the "Extending" guide's documentation rule,
 * which holds only with a dense 1024 x 1024 matrix per layer). Each token's
 * heads are flattened head-major, k = h * D + d (F = H * D), and mapped by one
 * dense real F x F matrix:
 *
 *   z[m, o] = sum_k W[o, k] * y[m, k]          (z = y W^T, no bias)
 *
 *   y        (tokens, H, D) float32: the scan output, tokens = batch * T.
 *   W        (F, F) float32, row-major: row o holds the weights of output o
 *            (the layout of a linear layer's weight); the block
 *            W[i*D:(i+1)*D, j*D:(j+1)*D] links head j to head i.
 *   z        out: (tokens, H, D) float32; must not overlap y or W
 *            (SSD_ERR_ALIAS).
 *   tokens   >= 0; with 0 nothing is launched and y, W, z may be NULL.
 *            H, D >= 1; D <= 256; H * D <= 16384.
 * Arithmetic: float32 products summed in float32 (fp32 MFMA).
 * Alignment: 4 bytes (16-byte aligned y and W with H * D % 4 == 0 take the
 * vector loads).
 * Status: SSD_ERR_SHAPE for sizes out of range, SSD_ERR_BLOCK_DIMS for D > 256,
 * SSD_ERR_UNSUPPORTED for H * D > 16384.
 */
int ssd_head_mix(const float *y, const float *W, int64_t tokens, int64_t H, int64_t D, float *z,
                 ssd_stream_t stream);

/* Workspace bytes that ssd_head_mix_backward needs (0 for invalid sizes, for
 * tokens == 0, and when the weight gradient is formed in one pass). It holds
 * partial weight gradients over token ranges: at most 256 * (H*D)^2 * 4 bytes,
 * 64 MiB at H * D = 1024 with 65,536 tokens. */
size_t ssd_head_mix_backward_workspace_bytes(int64_t tokens, int64_t H, int64_t D);

/*
 * ssd_head_mix_backward -- gradients of l = sum grad_z * z for ssd_head_mix,
 * by the chain rule on its definition:
 *
 *   grad_y[m, k] = sum_o grad_z[m, o] * W[o, k]      (grad_y = grad_z W)
 *   grad_W[o, k] = sum_m grad_z[m, o] * y[m, k]      (grad_W = grad_z^T y)
 *
 *   y, W, tokens, H, D  as for ssd_head_mix (y is the forward's input).
 *   grad_z    (tokens, H, D) float32.
 *   grad_y    out: (tokens, H, D) float32.
 *   grad_W    out: (F, F) float32, overwritten. The sum over tokens runs in a
 *             fixed order: repeated calls give identical bits. With tokens == 0
 *             it is set to zero and every other pointer may be NULL.
 *   workspace device memory of ssd_head_mix_backward_workspace_bytes bytes,
 *             256-byte aligned (NULL allowed when that is 0).
 * No output may overlap an input, each other or the workspace (SSD_ERR_ALIAS).
 * Alignment and status codes as ssd_head_mix; SSD_ERR_WORKSPACE when the
 * workspace is missing or too small.
 */
int ssd_head_mix_backward(const float *y, const float *W, const float *grad_z, int64_t tokens,
                          int64_t H, int64_t D, float *grad_y, float *grad_W, void *workspace,
                          size_t workspace_bytes, ssd_stream_t stream);

/* Static text for a status code (never NULL). */
const char *ssd_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int ssd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
