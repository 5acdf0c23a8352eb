/*
 * liblq: the LiftQuant lift-then-project decode operator on AMD Instinct
 * MI355X (gfx950), behind a plain C ABI.
 *
 * The operator (LiftQuant, arXiv 2606.04050, "LiftQuant: Continuous Bit-Width
 * LLM via Dimensional Lifting and Projection"; §3 introduction and §3.1 of
 * the paper, and the Method paragraph of the paper review of the same title):
 *
 *   A weight row of length K is cut into Kb = ceil(K/d) blocks of d weights.
 *   Block b is stored as D one-bit signs w_q in {+1,-1}^D and decoded as
 *   w = M w_q with one shared d x D mapping matrix M, so a layer costs
 *   N * Kb * D bits (D/d bits per weight). The decode computes
 *
 *       y = diag(s) W (M T a)
 *
 *   for activations a: T is a whitening transform (Hadamard mixing plus
 *   per-channel scaling), M lifts each d-block of T a into D-space,
 *   z_b = M^T (T a)_b, W is the N x L sign matrix (L = Kb * D) and s is a
 *   per-row scale. In this library:
 *
 *       xt = T x,   T = blockdiag_q(H_hb diag(c_q)),  H_hb orthonormal
 *                       Sylvester-ordered Hadamard of order hb
 *       z[b*D + e] = sum_i M[i][e] * xt[b*d + i]   (xt zero for k >= K)
 *       y[n] = row_scale[n] * sum_j S[n][j] * z[j]
 *
 * Conventions shared by every entry point:
 *
 *   - Pointers to tensors are DEVICE pointers owned by the caller, unless the
 *     argument says "host". The library allocates no memory and keeps no
 *     pointer after a call returns. Tensors are dense, row-major, and must be
 *     16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it asynchronously; results are valid once the
 *     stream has reached that point. Inputs must stay unchanged until then.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On any error the call returns a non-zero lq_status, enqueues nothing
 *     and writes nothing. B == 0 (or N == 0) is a valid empty call that
 *     enqueues nothing.
 *   - Results are deterministic: equal inputs give bitwise equal outputs on
 *     the same GPU (no floating-point atomics).
 *   - Functions never throw; they are thread-safe. Calls that share a
 *     workspace buffer must be ordered by the caller.
 *   - Workspaces: the first LQ_WS_CONTROL_BYTES bytes of a workspace hold
 *     control words through which the workgroups of the one-launch decodes
 *     (LQ_ALGO_FUSED, LQ_ALGO_FUSED_SPLIT) order themselves. Before its first use a workspace
 *     must be zero-filled (allocate it zeroed, or call lq_workspace_init);
 *     afterwards the library keeps those words consistent from call to call,
 *     and the caller must not write them. After LQ_ERR_HIP or a device fault,
 *     prepare the workspace again.
 *
 * Packed sign layout (this library's format; the pages give none). S is
 * N x L, N % 16 == 0, L % 8 == 0, total exactly N * L / 8 bytes:
 *   - panel p = rows 16p..16p+15 occupies bytes [p*2L, (p+1)*2L);
 *   - the first L/512 column tiles of a panel are 1024-byte full tiles; in
 *     tile q the 16-byte slot l = 16*g + r (g < 4, r < 16) belongs to row
 *     16p + r and its little-endian 32-bit word u (u < 4) holds, in bit b,
 *     column q*512 + 128*u + 32*g + b;
 *   - the remaining L % 512 columns (m = (L % 512) / 8 bytes per row) follow
 *     as a row-major tail: byte t of row r at r*m + t, bit e = column
 *     (L/512)*512 + 8t + e;
 *   - a set bit is the sign -1.
 */
#ifndef LIFTQUANT_LQ_H
#define LIFTQUANT_LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lq_status {
  LQ_OK = 0,
  LQ_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, negative size, d > D, ... */
  LQ_ERR_UNSUPPORTED = 2,   /* valid maths but outside this library's limits */
  LQ_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
  LQ_ERR_HIP = 4,           /* a HIP runtime call failed; see lq_last_hip_error */
  LQ_ERR_DEVICE = 5         /* a kernel reported a failure of its own (only the
                               one-launch decode LQ_ALGO_FUSED can: see
                               lq_workspace_status); that call's output is wrong */
} lq_status;

typedef enum lq_dtype {
  LQ_F32 = 0,               /* IEEE binary32 */
  LQ_BF16 = 1               /* bfloat16 (upper half of binary32), RNE conversion */
} lq_dtype;

/* Sign-product algorithm for lq_sign_gemm_ex. */
typedef enum lq_algo {
  LQ_ALGO_AUTO = 0,         /* the library's choice (what lq_sign_gemm does) */
  LQ_ALGO_VALU = 1,         /* fp32 sign-select on the vector ALUs; any z dtype,
                               B <= 16 per pass; exact fp32 accumulation */
  LQ_ALGO_MFMA_SMALL = 2,   /* B <= 16: packed signs fed to the FP4 x FP6
                               matrix cores as bit planes; z carried as a sum of
                               FP6 (E2M3) residual terms with a power-of-two
                               scale per 32-value block (4 terms for fp32 z, 3
                               beyond B = 12; 2 for bf16 z: about 2^-20, 2^-15
                               and 2^-10 of the block's largest magnitude);
                               fp32 accumulate */
  LQ_ALGO_MFMA_LARGE = 3,   /* any B: tiled GEMM on bf16 matrix cores, z as bf16
                               (bf16 z) or as a bf16 hi+lo pair (fp32 z) */
  LQ_ALGO_FUSED = 4,        /* lq_linear_ex only: the whole operator in ONE
                               launch, the MFMA_SMALL arithmetic (same FP6
                               terms, same results up to fp32 summation order):
                               the first workgroups whiten and lift x and
                               publish the activation operand, every workgroup
                               streams its weight panels meanwhile. Applies
                               when the operand fits one 16-column set
                               (B <= 8 bf16 x, B <= 4 fp32 x) and
                               ceil(L/512)*B is at most both the number of
                               workgroups and of compute units; otherwise
                               UNSUPPORTED */
  LQ_ALGO_FUSED_LOCAL = 5,  /* lq_linear_ex only, batch 1: the whole operator
                               in ONE launch with no communication between
                               workgroups: each prepares the whole activation
                               operand in LDS (same arithmetic as MFMA_SMALL)
                               and multiplies its 4 panels. Applies when
                               K <= 8192, d <= 16, L <= 10240 (+ tail) and the
                               operand fits LDS; otherwise UNSUPPORTED. Needs
                               no workspace */
  LQ_ALGO_WSPACE = 6,       /* lq_linear_ex only, bf16 x, any B: the product in
                               W space ([paper] §3: the weights a block's signs
                               represent are M times the sign vector). The
                               dense weights W[n][b*d+i] = sum_e M[i][e] s_e
                               are rebuilt per block on the fly (fp32 sums in
                               order of e, rounded to bf16), and bf16 matrix
                               cores reduce over the d*ceil(K/d) inputs
                               (transformed x rounded to bf16) instead of the
                               L lifted columns: D/d times fewer MACs. Applies
                               when D is 4 or 8 and d <= 4; otherwise (and for
                               fp32 x) UNSUPPORTED */
  LQ_ALGO_FUSED_SPLIT = 7   /* lq_linear_ex only, batch 1: the whole operator
                               in ONE launch split over the reduction: each
                               workgroup whitens, lifts and converts (the
                               MFMA_SMALL arithmetic) only the <= 6 column
                               tiles of its tile group, for its 16 panels;
                               the tile groups' partial row sums are added by
                               the group's last workgroup in a fixed order
                               (deterministic), through the workspace and a
                               ticket per 16-panel group in its control area
                               (reset by that workgroup: calls sharing a
                               workspace must not overlap). Applies when
                               d <= 16, D <= 32, d*D <= 512, at least one full
                               tile, the whitened span of a group <= 5120
                               inputs and N <= 262144; otherwise UNSUPPORTED */

} lq_algo;

/* Limits. d and D are runtime parameters: one operator for every rate. */
#define LQ_MAX_D 64          /* 1 <= d <= D <= LQ_MAX_D */
#define LQ_MAX_L (1 << 28)   /* lifted columns per row, L = ceil(K/d) * D */
#define LQ_MAX_HB 1024       /* hb a power of two, 1 <= hb <= 1024, hb | K */

/* Workspace control area (see the conventions above). */
#define LQ_WS_CONTROL_BYTES 20992
/* 32-bit word of the control area that the one-launch decode sets non-zero
 * when a workgroup gave up waiting for the activation operand (about one
 * second; possible only when other work holds the GPU's compute units): the
 * output of that call is then wrong. lq_workspace_init clears it. */
#define LQ_WS_ERROR_WORD 96

/* One quantized linear layer (all pointers device, caller-owned). */
typedef struct lq_layer {
  int64_t N;                 /* output features, N % 16 == 0 */
  int64_t K;                 /* input features, K % hb == 0 */
  int32_t d;                 /* block length */
  int32_t D;                 /* lifted dimension, ceil(K/d)*D % 8 == 0 */
  int32_t hb;                /* Hadamard block of T */
  int32_t reserved;          /* must be 0 */
  const uint8_t* packed;     /* N*ceil(K/d)*D/8 bytes, layout above */
  const float* M;            /* d x D, row-major */
  const float* c;            /* K channel scales of T */
  const float* row_scale;    /* N row scales (the paper's diag(s)) */
} lq_layer;

/* Library version, major*10000 + minor*100 + patch. Host only. */
int lq_version(void);

/* Human-readable name of a status code (static string). Host only. */
const char* lq_status_string(lq_status status);

/* hipError_t of the last LQ_ERR_HIP returned on this thread (0 if none). */
int lq_last_hip_error(void);

/*
 * Storage of one layer: *bytes = N * ceil(K/d) * D / 8 (every weight block
 * costs exactly D bits; paper §3 introduction and §3.1). Host only; `bytes`
 * is a host pointer. Errors: INVALID_ARG for N < 0, K < 1, d < 1, D < d,
 * null bytes; UNSUPPORTED for D > LQ_MAX_D, N % 16 != 0 or L % 8 != 0.
 */
lq_status lq_packed_size(int64_t N, int64_t K, int32_t d, int32_t D, size_t* bytes);

/*
 * Pack signs into the layout above.
 * signs:  int8, N x Kb x D (= N x L row-major), every entry +1 or -1
 *         (any negative value packs as -1, anything else as +1).
 * packed: lq_packed_size bytes, fully overwritten.
 * The signs are the w_q of every block (paper §3.1; one-bit weights of the
 * INT1 GEMM, review Method and Released resources).
 */
lq_status lq_pack_signs(const int8_t* signs, int64_t N, int64_t K, int32_t d, int32_t D,
                        uint8_t* packed, void* stream);

/* Inverse of lq_pack_signs: writes N x L int8 values +1/-1. */
lq_status lq_unpack_signs(const uint8_t* packed, int64_t N, int64_t K, int32_t d, int32_t D,
                          int8_t* signs, void* stream);

/*
 * Whitening xt = T x (paper §3 introduction, the layer-wise whitening T;
 * review Method: Hadamard mixing plus scalings), with
 * T = blockdiag_q(H_hb diag(c_q)): for every batch row and every run of hb
 * channels, xt = H_hb (c .* x) with H_hb[i][j] = (-1)^popcount(i&j)/sqrt(hb).
 * x: B x K in xtype (F32 or BF16); c: K floats; xt: B x K floats.
 * hb == 1 applies only the channel scales. Computed in fp32.
 */
lq_status lq_hadamard_scale(const void* x, lq_dtype xtype, int64_t B, int64_t K, int32_t hb,
                            const float* c, float* xt, void* stream);

/*
 * Lift: z[b][j*D + e] = sum_{i<d} M[i][e] * xt[b][j*d + i], with xt taken as
 * zero for columns k >= K (the virtual zero pad to Kb*d). This is the M T a
 * factor of the fused operator (paper §3 introduction). xt: B x K floats;
 * M: d x D floats; z: B x L in ztype (F32 or BF16, RNE). fp32 arithmetic.
 */
lq_status lq_lift_activations(const float* xt, int64_t B, int64_t K, int32_t d, int32_t D,
                              const float* M, void* z, lq_dtype ztype, void* stream);

/*
 * Sign product with row scale: y[b][n] = row_scale[n] * sum_j S[n][j] z[b][j]
 * (the INT1 x FP GEMM of the decode path, review Method; diag(s) of the
 * paper's fused operator, §3 introduction).
 * packed: N x L signs, layout above; z: B x L in ztype; row_scale: N floats;
 * y: B x N in ytype. ws: device workspace of at least
 * lq_sign_gemm_workspace_size bytes (may be NULL when that size is 0).
 * lq_sign_gemm uses LQ_ALGO_AUTO. Accumulation is fp32 on every algorithm.
 */
lq_status lq_sign_gemm_workspace_size(int64_t B, int64_t N, int64_t L, lq_dtype ztype,
                                      lq_algo algo, size_t* bytes);
lq_status lq_sign_gemm(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B,
                       int64_t N, int64_t L, const float* row_scale, void* y, lq_dtype ytype,
                       void* ws, size_t ws_bytes, void* stream);
lq_status lq_sign_gemm_ex(const uint8_t* packed, const void* z, lq_dtype ztype, int64_t B,
                          int64_t N, int64_t L, const float* row_scale, void* y, lq_dtype ytype,
                          lq_algo algo, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole decode operator y = diag(s) W (M T x) (paper §3 introduction):
 * whitening, lift and sign product in sequence on `stream`.
 * x: B x K in xtype; y: B x N in ytype. fp32 activations keep fp32 lifted
 * values end to end; bf16 activations use bf16 lifted values on the matrix
 * cores. ws: device workspace of at least lq_linear_workspace_size bytes.
 */
lq_status lq_linear_workspace_size(const lq_layer* layer, int64_t B, lq_dtype xtype,
                                   size_t* bytes);
lq_status lq_linear(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B, void* y,
                    lq_dtype ytype, void* ws, size_t ws_bytes, void* stream);

/*
 * As lq_linear, with the algorithm chosen by the caller: LQ_ALGO_AUTO (what
 * lq_linear does: B > 16: WSPACE for bf16 x where it applies, else
 * MFMA_LARGE; B <= 16: fp32 x VALU, bf16 x MFMA_SMALL), VALU (B <= 16),
 * MFMA_SMALL (B <= 16; whitening, lift and operand in one preparation
 * launch, then the product launch), MFMA_LARGE, FUSED, FUSED_LOCAL or WSPACE
 * (UNSUPPORTED where they do not apply).
 * The workspace size depends on the algorithm.
 */
lq_status lq_linear_workspace_size_ex(const lq_layer* layer, int64_t B, lq_dtype xtype,
                                      lq_algo algo, size_t* bytes);

/*
 * The algorithm lq_linear_ex(layer, ., xtype, B, ., ., algo, ...) runs
 * (AUTO resolved), written to *resolved; host-only, launches nothing.
 * Errors: as lq_linear_workspace_size_ex, and INVALID_ARG for B < 1.
 */
lq_status lq_linear_algo(const lq_layer* layer, int64_t B, lq_dtype xtype, lq_algo algo,
                         lq_algo* resolved);
lq_status lq_linear_ex(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B, void* y,
                       lq_dtype ytype, lq_algo algo, void* ws, size_t ws_bytes, void* stream);

/*
 * How a call would run, without running it (host only, launches nothing):
 * the algorithm (AUTO resolved) and the shape of its sign-product launch,
 * the one kernel that streams the packed signs (the decode's INT1 x FP GEMM,
 * review Method). lq_linear_plan takes lq_linear_ex's arguments,
 * lq_sign_gemm_plan lq_sign_gemm_ex's. Errors: as lq_linear_algo (and as
 * lq_sign_gemm_workspace_size for lq_sign_gemm_plan), INVALID_ARG for a NULL
 * info or B < 1.
 */
typedef struct lq_plan_info {
  int32_t algo;              /* the lq_algo that runs */
  int32_t workgroups;        /* workgroups of the sign-product launch */
  int32_t waves;             /* wavefronts per workgroup of that launch */
  int32_t panels;            /* 16-row panels of S per workgroup */
  int32_t batch_rows;        /* batch rows per workgroup */
  int32_t ksplit;            /* workgroups that share the same output rows, each
                                multiplying a part of the reduction (1 = none) */
} lq_plan_info;
lq_status lq_linear_plan(const lq_layer* layer, int64_t B, lq_dtype xtype, lq_algo algo,
                         lq_plan_info* info);
lq_status lq_sign_gemm_plan(int64_t B, int64_t N, int64_t L, lq_dtype ztype, lq_algo algo,
                            lq_plan_info* info);

/*
 * Whether the calls that used a workspace ran correctly: waits for `stream`
 * (hipStreamSynchronize; not while it is being captured), then reads the
 * control area's error word. LQ_ERR_DEVICE when it is set: a one-launch
 * decode (LQ_ALGO_FUSED, [paper] §3 introduction: the whole operator in one
 * kernel) gave up waiting for the activation operand, so the output of that
 * call is wrong; the word stays set until lq_workspace_init. LQ_OK otherwise,
 * and for workspaces shorter than LQ_WS_CONTROL_BYTES (no call that can fail
 * this way uses those). Errors: INVALID_ARG for a NULL or unaligned ws with
 * ws_bytes >= LQ_WS_CONTROL_BYTES; LQ_ERR_HIP if the copy or the wait fails.
 */
lq_status lq_workspace_status(const void* ws, size_t ws_bytes, void* stream);

/*
 * Test aid for that failure path: while `enable` is non-zero, the loaders of
 * LQ_ALGO_FUSED launches wait for a publication that no producer makes,
 * polling only a few times, so every one of them gives up at once and sets
 * the error word; every kernel still runs to its end and the control words
 * stay consistent for the next launch (the outputs of those calls are wrong
 * by construction). Process-wide; 0 restores the normal waits. Host only.
 */
lq_status lq_debug_fused_timeout(int32_t enable);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): lq_linear
 * without a caller workspace. It runs exactly what lq_linear runs (the same
 * algorithm, kernels and results) with the workspace carved from a
 * file-scope device array of LQ_NOALLOC_SCRATCH_BYTES bytes inside the
 * library: one array per GPU, whose address the first call on a GPU looks up
 * (with that GPU current) and keeps; each GPU holds it until the process
 * ends. Nothing is allocated and no allocating routine is called.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (each call rewrites everything it reads from it): calls that
 * overlap on one GPU race, so order them (one stream, or events between
 * streams). Errors: as lq_linear; UNSUPPORTED when lq_linear's workspace for
 * this call would exceed LQ_NOALLOC_SCRATCH_BYTES (checked on the host
 * before anything is enqueued), LQ_ERR_HIP when the array's address cannot
 * be looked up.
 */
#define LQ_NOALLOC_SCRATCH_BYTES (16u << 20)
lq_status lq_linear_noalloc(const lq_layer* layer, const void* x, lq_dtype xtype, int64_t B,
                            void* y, lq_dtype ytype, void* stream);

/*
 * Several layers on the same input (as the gate and up projections of a
 * transformer MLP): ys[i] = lq_linear(&layers[i], x) for i < n, with
 * 1 <= n <= LQ_MULTI_MAX and every layer of the same K (d, D, hb, M, c and N
 * may differ). Where lq_linear would run the small-batch matrix-core path
 * (MFMA_SMALL) for every layer (B <= 16, bf16 x) and the layers' product
 * plans agree once the panels per workgroup are chosen for all their panels
 * together (layers of the same shape do), the n operands come from one
 * preparation launch and the n products from one product launch: the same
 * arithmetic as lq_linear, its fp32 partial sums split among wavefronts as
 * that choice of panels per workgroup gives (bit-for-bit lq_linear's result
 * where the choice is the single call's, else within fp32 rounding of it).
 * Otherwise the layers run one after another as n lq_linear calls.
 * ys: host array of n device pointers (B x N_i in ytype each).
 * ws: device workspace of at least lq_linear_multi_workspace_size bytes.
 * Errors: as lq_linear, and INVALID_ARG for NULL layers or ys, n outside
 * [1, LQ_MULTI_MAX] or layers of different K.
 */
#define LQ_MULTI_MAX 4
lq_status lq_linear_multi_workspace_size(const lq_layer* layers, int32_t n, int64_t B,
                                         lq_dtype xtype, size_t* bytes);
lq_status lq_linear_multi(const lq_layer* layers, int32_t n, const void* x, lq_dtype xtype,
                          int64_t B, void* const* ys, lq_dtype ytype, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Prepare a workspace for first use: zero-fill its control area (the first
 * min(ws_bytes, LQ_WS_CONTROL_BYTES) bytes, with a kernel on `stream`).
 * Errors: INVALID_ARG for a NULL or unaligned ws with ws_bytes > 0.
 */
lq_status lq_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Nearest-neighbour encoding ([paper] §3.1, Eq. (1): the inner minimisation,
 * which the paper names the nearest-neighbour search, i.e. the quantization
 * step): for every d-block w_b,
 *     s_b = argmin over s in {+1,-1}^D of || w_b - M s ||_2,
 * searched exhaustively over the 2^D sign vectors (fp64 residuals); among
 * equally close vectors the one with the lowest index, index bit e set
 * meaning s_e = -1.
 * w: nblocks x d floats (device; for a weight matrix already in the lifted
 * model's frame, its rows' d-blocks in order), M: d x D floats (device),
 * signs: nblocks x D int8 (device, +1 / -1: the input of lq_pack_signs),
 * dist2: nblocks floats (device, may be NULL): the squared distance.
 * Limits: 1 <= d <= LQ_ENCODE_MAX_SMALL_D, d <= D <= LQ_ENCODE_MAX_D
 * (UNSUPPORTED beyond). Errors: INVALID_ARG for NULL pointers with
 * nblocks > 0, float pointers not 4-byte aligned, nblocks < 0 or d > D.
 */
#define LQ_ENCODE_MAX_D 24
#define LQ_ENCODE_MAX_SMALL_D 16
lq_status lq_encode(const float* w, int64_t nblocks, int32_t d, int32_t D, const float* M,
                    int8_t* signs, float* dist2, void* stream);

/*
 * The nearest-neighbour search of lq_encode reduced from 2^D to 2^(D-d) sign
 * vectors by pseudo-inverse initialisation ([review] Method: encoding
 * "accelerated from 2^D to 2^(D-d)"; [review] Limitations: the exhaustive
 * search is practically capped at D - d <= 20). Reading: M = [M_a | M_f],
 * the first d columns solved for, the other D - d enumerated; for every sign
 * vector s_f of M_f, s_a = sgn(M_a^-1 (w - M_f s_f)) (+1 at 0), the candidate
 * s = (s_a, s_f); the candidate closest to w_b wins (fp64 residuals), among
 * equally close ones the lowest index (index bit e set meaning s_e = -1).
 * Exact (lq_encode's result) when M_a is diagonal; otherwise never closer
 * than lq_encode. Makes LQ-32/16 (2^16 candidates per block) encodable.
 * w, M, signs, dist2: as lq_encode. ws: device workspace of
 * lq_encode_pinv_workspace_size bytes (16-byte aligned): the tables
 * M_a^-1 and M_a^-1 M_f (fp64), computed on the host: the call copies M to
 * the host and synchronizes `stream` twice (M read, tables written) before
 * the search kernel is enqueued.
 * Limits: 1 <= d <= LQ_ENCODE_MAX_SMALL_D, d <= D <= LQ_ENCODE_PINV_MAX_D,
 * D - d <= LQ_ENCODE_PINV_MAX_FREE (UNSUPPORTED beyond). Errors: as
 * lq_encode; INVALID_ARG also when M_a is singular (a pivot of its
 * elimination at most 2^-40 of its largest magnitude) or ws is not 16-byte
 * aligned; WORKSPACE for a missing or short workspace.
 */
#define LQ_ENCODE_PINV_MAX_D 32
#define LQ_ENCODE_PINV_MAX_FREE 24
lq_status lq_encode_pinv_workspace_size(int32_t d, int32_t D, size_t* bytes);
lq_status lq_encode_pinv(const float* w, int64_t nblocks, int32_t d, int32_t D, const float* M,
                         int8_t* signs, float* dist2, void* ws, size_t ws_bytes, void* stream);

/*
 * One gradient step on M of the objective of [paper] §3.1 Eq. (1), on the
 * caller's samples w (n x d floats on the device, drawn from N(0, I_d)):
 *     loss(M) = mean_b min_s || w_b - M s ||_2     (the norm as printed).
 * The minimiser s_b* (lq_encode's) is piecewise constant in M, so the
 * gradient of the minimum is that of ||w_b - M s_b*|| with s_b* held fixed,
 * -(r_b / ||r_b||) s_b*^T, r_b = w_b - M s_b* (zero where r_b = 0); the step
 * is M <- M - lr * (its mean over the samples), in fp64, stored back into M
 * (d x D floats, device, in place). loss: one float (device, may be NULL):
 * the loss at the old M. Deterministic: fixed summation order.
 * ws: device workspace of lq_train_m_step_workspace_size bytes (16-byte
 * aligned). Limits as lq_encode. Errors: as lq_encode, WORKSPACE for a
 * missing or short workspace.
 */
lq_status lq_train_m_step_workspace_size(int64_t n, int32_t d, int32_t D, size_t* bytes);
lq_status lq_train_m_step(float* M, const float* w, int64_t n, int32_t d, int32_t D, float lr,
                          float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * Profiling aid: time the sign-product kernel itself. `starts` and `stops`
 * are host arrays of `count` hipEvent_t handles (passed as void*) created by
 * the caller. While set, every sign-product kernel launched by lq_sign_gemm,
 * lq_sign_gemm_ex, lq_linear or lq_linear_ex (for LQ_ALGO_FUSED, the one
 * kernel of the call) records starts[i] and stops[i] at its own
 * start and end (the events ride on the kernel's dispatch, as in
 * hipExtLaunchKernelGGL, so they time the kernel alone, as a profiler does),
 * i = 0, 1, 2, ... wrapping modulo `count` (the preparation kernels are not
 * timed). Do not set the ring while capturing a stream into a graph. count == 0 clears the ring (the
 * arrays may then be NULL); calling again restarts at slot 0. The ring is
 * process-wide and guarded by a lock; the caller keeps the events alive
 * while it is set. Errors: INVALID_ARG for count < 0 or NULL arrays with
 * count > 0.
 */
lq_status lq_profile_events(void* const* starts, void* const* stops, int32_t count);

#ifdef __cplusplus
}
#endif

#endif /* LIFTQUANT_LQ_H */
