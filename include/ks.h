/*
 * ks.h -- C ABI of libks: Kronecker-sparse (KS) matrix multiplication on
 * AMD MI355X (gfx950).
 *
 * The operation. A KS matrix has a support that is a Kronecker product of
 * identity and all-ones blocks (KS abstract page, taxoreview.com
 * "dblp:303/4794", first paragraph, first sentence). libks handles the
 * support I_a (x) 1_{b x c} (x) I_d: W is (a*b*d) x (a*c*d) and holds
 * a*b*c*d nonzeros, stored densely as a 4-D tensor K of shape (a, d, b, c),
 * gamma fastest, with
 *     W[alpha*b*d + beta*d + delta][alpha*c*d + gamma*d + delta]
 *         = K[alpha][delta][beta][gamma].
 * Every entry point computes Y = X * W^T for a batch of rows:
 *     Y[n][alpha][beta][delta] = sum_gamma K[alpha][delta][beta][gamma]
 *                                        * X[n][alpha][gamma][delta],
 * X is batch x (a*c*d) and Y is batch x (a*b*d), both row-major, batch first.
 * The same page's third paragraph factorises matrices into products of
 * butterfly-support factors, and its first sentence ties KS matrices to
 * Butterfly and Monarch matrices, which are such products: ks_chain_matmul
 * applies a list of factors in order. The page's third sentence describes
 * the kernel principle followed here: one fused pass, output-stationary,
 * with no separate permutation of X or Y through global memory.
 *
 * Conventions for every entry point.
 *  - All tensor pointers (W, X, Y, workspace) are DEVICE pointers owned by
 *    the caller. libks never allocates or frees device memory and keeps no
 *    per-call state; it is safe to call from several host threads.
 *  - Calls are asynchronous on `stream` (0 = the null stream). Argument
 *    errors are detected on the host before any HIP call and returned as a
 *    status; nothing is launched then. Launch failures are returned as
 *    KS_ERR_HIP. Faults during execution surface at the caller's next
 *    synchronisation, as for any HIP kernel.
 *  - batch == 0 is a valid no-op.
 *  - Results are deterministic: the same call on the same inputs gives
 *    bit-identical outputs (no atomics, fixed summation order per kernel).
 *  - No exception crosses the ABI.
 */
#ifndef KS_H_
#define KS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The KS pattern (a, b, c, d): support I_a (x) 1_{b x c} (x) I_d.
 * Each field must be >= 1 (powers of two are not required). n_in = a*c*d,
 * n_out = a*b*d and nnz = a*b*c*d must each be below 2^31. */
typedef struct ks_pattern_t {
    int32_t a, b, c, d;
} ks_pattern_t;

/* Element types. Accumulation is always fp32 and Y is always fp32.
 *  KS_DTYPE_F32   X fp32,  W fp32.
 *  KS_DTYPE_BF16  X bf16,  W bf16 (products of two bf16 values are exact
 *                 in fp32, so only the fp32 accumulation rounds).
 *  KS_DTYPE_BF16W X fp32,  W bf16 (the later factors of a bf16 chain, whose
 *                 inputs are fp32 intermediates).
 * bf16 is the upper 16 bits of an IEEE fp32 word. */
typedef enum ks_dtype_t {
    KS_DTYPE_F32 = 0,
    KS_DTYPE_BF16 = 1,
    KS_DTYPE_BF16W = 2
} ks_dtype_t;

typedef enum ks_status_t {
    KS_OK = 0,
    KS_ERR_NULL = 1,            /* a required pointer is NULL (batch > 0)      */
    KS_ERR_PATTERN = 2,         /* a field < 1, or n_in/n_out/nnz >= 2^31      */
    KS_ERR_BATCH = 3,           /* batch < 0 or batch >= 2^31                  */
    KS_ERR_DTYPE = 4,           /* unknown dtype                               */
    KS_ERR_CHAIN_MISMATCH = 5,  /* n < 1, or n_out(p[k]) != n_in(p[k+1])       */
    KS_ERR_WORKSPACE = 6,       /* workspace NULL or smaller than required     */
    KS_ERR_ALIGN = 7,           /* pointer not aligned to its element size     */
    KS_ERR_OVERLAP = 8,         /* Y (or workspace) overlaps an input          */
    KS_ERR_HIP = 9,             /* a HIP call failed (launch, device query)    */
    KS_ERR_UNSUPPORTED = 10,    /* a forced kernel cannot run this pattern     */
    KS_ERR_INVALID = 11         /* other invalid argument (flags, options)     */
} ks_status_t;

/* Kernel families, for ks_matmul_ex (tests and benchmarks only). */
typedef enum ks_kernel_t {
    KS_KERNEL_AUTO = 0,     /* the planner's choice (what ks_matmul runs)        */
    KS_KERNEL_GENERIC = 1,  /* one thread per output, any pattern                */
    KS_KERNEL_VALU = 2,     /* weights in registers, fp32 FMA (b, c <= 16)       */
    KS_KERNEL_MFMA = 3,     /* matrix cores (b, c >= 16), LDS-staged tiles       */
    KS_KERNEL_MFMA_LDS = 4, /* same kernels as KS_KERNEL_MFMA (kept for ABI)     */
    KS_KERNEL_COLUMN = 5    /* matrix cores, output computed in place in the
                               staged X tile: b = c in {16, 32}, d a multiple
                               of 32 (b = 16) or 16 (b = 32), fp32 X           */
} ks_kernel_t;

/* Who stores Y in the MFMA kernels, for ks_options_t.store_waves. */
typedef enum ks_store_waves_t {
    KS_STORE_AUTO = 0,      /* the planner's choice                              */
    KS_STORE_COMPUTE = 1,   /* the compute waves, after each step's MFMAs        */
    KS_STORE_DEDICATED = 2  /* a storer wave, overlapped with the next step's
                               MFMAs (needs LDS for two Y tiles)                 */
} ks_store_waves_t;

/* Tile candidates of the matrix-core kernel: k = 1..KS_MFMA_TILES selects
   (B-operand register budget, b split) = (32, 1), (64, 1), (128, 1),
   (128, 2), (64, 2), (128, 4), (64, 4) for the k-th entry. */
#define KS_MFMA_TILES 7

typedef struct ks_options_t {
    int32_t kernel;         /* a ks_kernel_t value                               */
    int32_t rows_per_block; /* 0 = planner default; else rows per workgroup step */
    int32_t store_waves;    /* a ks_store_waves_t value; MFMA family only;
                               KS_ERR_UNSUPPORTED if the tile cannot use it      */
    int32_t mfma_tile;      /* 0 = planner choice; 1..KS_MFMA_TILES forces that
                               tile candidate (MFMA family only);
                               KS_ERR_UNSUPPORTED if it does not fit the pattern */
    int32_t mfma_loaders;   /* 0 = planner choice; 1 or 2 waves streaming X into
                               LDS (MFMA family only; 2 needs c >= 64, else
                               KS_ERR_UNSUPPORTED)                               */
    int32_t reserved[3];    /* must be zero                                      */
} ks_options_t;

/* Chain flags. */
#define KS_CHAIN_AUTO 0u      /* fuse consecutive factors where the planner can */
#define KS_CHAIN_NO_FUSE 1u   /* one launch per factor, through the workspace   */

/* Human-readable name of a status; never NULL. */
const char* ks_status_string(ks_status_t status);

/* Library version string, e.g. "libks 0.1.0 gfx950". */
const char* ks_version(void);

/*
 * ks_matmul: Y = X * W^T for one KS factor p.
 *   W      device, K tensor of shape (p.a, p.d, p.b, p.c), contiguous,
 *          element type per dt.
 *   X      device, batch x (a*c*d) row-major, element type per dt.
 *   Y      device, batch x (a*b*d) row-major fp32; fully overwritten.
 *   batch  number of rows, 0 <= batch < 2^31.
 *   dt     KS_DTYPE_F32, KS_DTYPE_BF16 or KS_DTYPE_BF16W.
 *   stream HIP stream for the launch.
 * Pointers must be aligned to their element size (4 bytes fp32, 2 bytes
 * bf16); 16-byte alignment enables wider loads but is not required.
 * Y must not overlap X or W (KS_ERR_OVERLAP).
 */
ks_status_t ks_matmul(ks_pattern_t p, const void* W, const void* X, void* Y,
                      int64_t batch, ks_dtype_t dt, hipStream_t stream);

/*
 * ks_matmul_ex: ks_matmul with options; opt may be NULL (same as ks_matmul).
 * opt->kernel forces a kernel family; KS_ERR_UNSUPPORTED if that family
 * cannot run p with dt. For tests and benchmarks that compare kernels on
 * the same input; results of every family agree within fp32 rounding.
 */
ks_status_t ks_matmul_ex(ks_pattern_t p, const void* W, const void* X, void* Y,
                         int64_t batch, ks_dtype_t dt, hipStream_t stream,
                         const ks_options_t* opt);

/*
 * Gradients of ks_matmul, for a layer's backward pass. The pages give the
 * layer (a KS linear layer usable from PyTorch: KS abstract page,
 * taxoreview.com "dblp:303/4794", first paragraph, last sentence); its
 * derivatives are the chain rule on Y = X * W^T. With dY = dL/dY
 * (batch x a*b*d):
 *   dX = dY * W     dX[n][alpha][gamma][delta]
 *                     = sum_beta K[alpha][delta][beta][gamma] dY[n][alpha][beta][delta]
 *   dK              dK[alpha][delta][beta][gamma]
 *                     = sum_n dY[n][alpha][beta][delta] X[n][alpha][gamma][delta]
 *
 * ks_matmul_dx_workspace_size: bytes of workspace ks_matmul_dx needs (W's
 *   blocks transposed: nnz elements of W's type, rounded up to 256), to
 *   *bytes. KS_ERR_NULL if bytes is NULL; pattern and dtype statuses as for
 *   ks_matmul.
 * ks_matmul_dx: dX = dY * W.
 *   W      device K tensor (a, d, b, c) as in ks_matmul.
 *   dY     device, batch x (a*b*d): fp32 for KS_DTYPE_F32 and KS_DTYPE_BF16W,
 *          bf16 for KS_DTYPE_BF16; W is bf16 for KS_DTYPE_BF16 and BF16W.
 *   dX     device fp32, batch x (a*c*d); fully overwritten.
 *   ws     device workspace, >= ks_matmul_dx_workspace_size bytes, 16-byte
 *          aligned (KS_ERR_WORKSPACE if NULL or smaller, KS_ERR_ALIGN).
 *   Runs as the forward product of pattern (a, c, b, d) with every block of
 *   W transposed (two launches on `stream`). dX must not overlap dY, W or
 *   ws, nor ws dY or W (KS_ERR_OVERLAP). batch = 0: nothing is launched.
 */
ks_status_t ks_matmul_dx_workspace_size(ks_pattern_t p, ks_dtype_t dt, size_t* bytes);
ks_status_t ks_matmul_dx(ks_pattern_t p, const void* W, const void* dY, void* dX, int64_t batch,
                         ks_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ks_matmul_dw_workspace_size: bytes of workspace ks_matmul_dw needs for
 *   this batch (0 if none; partial sums over ranges of rows), to *bytes.
 * ks_matmul_dw: dK (the gradient with respect to the K tensor).
 *   dY     device fp32, batch x (a*b*d).
 *   X      device, batch x (a*c*d): fp32 for KS_DTYPE_F32 and KS_DTYPE_BF16W,
 *          bf16 for KS_DTYPE_BF16 (the forward input).
 *   dW     device fp32, shape (a, d, b, c); fully overwritten (zeros when
 *          batch = 0).
 *   ws     device workspace of the queried size (may be NULL when 0),
 *          16-byte aligned.
 *   Partial sums over row ranges are added in a fixed order, so repeated
 *   calls give identical bits. dW must not overlap dY, X or ws, nor ws dY
 *   or X (KS_ERR_OVERLAP).
 */
ks_status_t ks_matmul_dw_workspace_size(ks_pattern_t p, int64_t batch, ks_dtype_t dt, size_t* bytes);
ks_status_t ks_matmul_dw(ks_pattern_t p, const void* dY, const void* X, void* dW, int64_t batch,
                         ks_dtype_t dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ks_matmul_dw_noalloc: ks_matmul_dw for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight training loops, harnesses
 * that forbid hipMalloc. It allocates nothing and takes no workspace: the
 * partial sums go to a scratch array of KS_DW_SCRATCH_BYTES that libks
 * keeps on every GPU it runs on until the process ends. Same arguments,
 * results (bit for bit: the same kernels and summation order) and statuses
 * as ks_matmul_dw without ws / ws_bytes; KS_ERR_WORKSPACE if the call would
 * need more scratch than KS_DW_SCRATCH_BYTES (the planner keeps every dK
 * call's partial sums within it, so this does not happen for valid
 * arguments). All calls on one GPU share its scratch: calls that overlap in
 * time on one GPU (several streams or host threads) race and give wrong
 * results; calls in sequence on one stream are safe.
 */
#define KS_DW_SCRATCH_BYTES (64u << 20)
ks_status_t ks_matmul_dw_noalloc(ks_pattern_t p, const void* dY, const void* X, void* dW, int64_t batch,
                                 ks_dtype_t dt, hipStream_t stream);

/*
 * ks_chain_workspace_size: bytes of device workspace ks_chain_matmul needs
 * for these arguments (0 if none), written to *bytes.
 *   p, n   the factors in application order (p[0] is applied to X first).
 *   dt     KS_DTYPE_F32, KS_DTYPE_BF16 or KS_DTYPE_BF16W (chain dtype: the
 *          types of X and of every W; intermediates are always fp32).
 *   flags  KS_CHAIN_AUTO or KS_CHAIN_NO_FUSE.
 * Returns the same validation statuses as ks_chain_matmul for p, n, batch,
 * dt and flags; KS_ERR_NULL if bytes is NULL.
 */
ks_status_t ks_chain_workspace_size(const ks_pattern_t* p, int n, int64_t batch,
                                    ks_dtype_t dt, unsigned flags, size_t* bytes);

/*
 * ks_chain_matmul: Y = X * (W_{n-1} ... W_1 W_0)^T, factor 0 applied first.
 *   p      host array of n patterns; n_out(p[k]) must equal n_in(p[k+1]).
 *   W      host array of n device pointers; W[k] holds factor k's K tensor
 *          (p[k].a, p[k].d, p[k].b, p[k].c).
 *   X      device, batch x n_in(p[0]); Y device fp32, batch x n_out(p[n-1]).
 *   dt     KS_DTYPE_F32: everything fp32. KS_DTYPE_BF16: X and every W are
 *          bf16; intermediates and Y are fp32, so factors after the first
 *          read fp32 inputs with bf16 weights. KS_DTYPE_BF16W: X fp32 and
 *          every W bf16 (the tail of a bf16 chain run on its own).
 *   ws     device workspace of ws_bytes >= ks_chain_workspace_size(...);
 *          may be NULL when that size is 0. 16-byte aligned. Must not
 *          overlap X, Y or any W.
 *   flags  KS_CHAIN_AUTO: consecutive factors whose joint tile fits on chip
 *          run as one fused launch with the intermediates kept in LDS.
 *          Scanning the chain from factor 0, at each factor the planner
 *          takes the first that applies of: the pair (1, b0, 16, 64) ->
 *          (b0, 8, 8, 8) with b0 % 8 == 0 (a group of beta0 needs whole
 *          rows of X and yields a slab of Y's row); the pair (a, 16, 16, 16)
 *          -> (16a, 16, 16, 1) (the second factor works inside the first
 *          one's per-alpha output slabs; the last two factors of the 16-ary
 *          butterfly); the longest run of at least two factors with blocks
 *          of b * c <= 16, at most 64 KB of weights each and rows of at most
 *          4096 elements, applied to whole rows held in LDS (radix-2 and
 *          radix-4 butterflies, Walsh-Hadamard products); else the factor
 *          alone. KS_CHAIN_NO_FUSE: one launch per factor. Results of the
 *          two modes agree to rounding.
 * All launches go to `stream` in order; there is no host synchronisation.
 */
ks_status_t ks_chain_matmul(const ks_pattern_t* p, int n, const void* const* W,
                            const void* X, void* Y, int64_t batch, ks_dtype_t dt,
                            void* ws, size_t ws_bytes, unsigned flags,
                            hipStream_t stream);

/*
 * ks_chain_plan: the launch groups ks_chain_matmul uses for these arguments.
 * Writes the number of groups to *groups and, for each group in order, the
 * number of consecutive factors it runs (1, or more for a fused group) to
 * group_len[0 .. min(*groups, cap) - 1]. Pure host code; no HIP call. Same
 * validation statuses as ks_chain_workspace_size; KS_ERR_NULL if groups is
 * NULL (group_len may be NULL when cap is 0).
 */
ks_status_t ks_chain_plan(const ks_pattern_t* p, int n, int64_t batch, ks_dtype_t dt,
                          unsigned flags, int* group_len, int cap, int* groups);

/*
 * ks_plan_describe: write a one-line description of the kernel and tile the
 * planner picks for (p, batch, dt) into buf (NUL-terminated, truncated to
 * len). Pure host code; no HIP call. For tests and benchmark labels.
 */
ks_status_t ks_plan_describe(ks_pattern_t p, int64_t batch, ks_dtype_t dt,
                             char* buf, size_t len);

/*
 * ks_pair_closure: the closure rule for running factor f and then factor g
 * in one pass, which the chain planner applies (KS abstract page, first
 * paragraph, first sentence: Butterfly and Monarch matrices are chains of
 * such factors). f's output groups (fixed alpha, delta of f; all beta) and
 * g's input groups (fixed alpha, delta of g; all gamma) link the
 * intermediate's n_out(f) values into closed components: a component's
 * outputs depend only on its own inputs, f blocks and g blocks. Reports the
 * component count, the largest component's sizes and the tile of components
 * whose X reads come in runs of 16 bytes (4 fp32 values). A pair can run
 * fused only if such a tile's intermediates fit in LDS and its weights near
 * the compute units; the planner also needs a kernel family for the shape.
 * Pure host code, no HIP call. KS_ERR_NULL (out), KS_ERR_PATTERN,
 * KS_ERR_CHAIN_MISMATCH (n_out(f) != n_in(g)), KS_ERR_UNSUPPORTED (an
 * intermediate of more than 2^22 values is not analysed).
 */
typedef struct ks_closure_t {
    int64_t components;       /* closed components of the intermediate */
    int64_t mid;              /* intermediate values of the largest component */
    int64_t inputs;           /* values of X it reads */
    int64_t outputs;          /* values of Y it writes */
    int64_t weights;          /* weights it needs: its blocks of f and of g */
    int64_t in_run;           /* shortest run of consecutive X indices it reads */
    int64_t out_run;          /* shortest run of consecutive Y indices it writes */
    int64_t tile_components;  /* components per tile with 16-byte X runs */
    int64_t tile_weights;     /* weights of such a tile */
    int32_t uniform;          /* 1: all components have the same size */
    int32_t reserved;         /* 0 */
} ks_closure_t;

ks_status_t ks_pair_closure(ks_pattern_t f, ks_pattern_t g, ks_closure_t* out);

/*
 * ks_chain_describe: one description per launch group of the chain
 * ks_chain_matmul would run for these arguments, "[first..last] kernel",
 * separated by "; ", into buf (NUL-terminated, truncated to len). Same
 * validation as ks_chain_plan; pure host code, no HIP call. Describes the
 * path for 16-byte-aligned X and Y (a group that needs them runs another
 * kernel otherwise). For tests and benchmark labels.
 */
ks_status_t ks_chain_describe(const ks_pattern_t* p, int n, int64_t batch, ks_dtype_t dt,
                              unsigned flags, char* buf, size_t len);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* KS_H_ */
