/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 int4 weight-only linear layer.
 *
 * The operation (LLM170, CUDA/W4A16 page, opening description): weights are
 * int4, symmetric (no zero point), with one fp16 scale per group of `group`
 * input features along K (128 for the dense model, 32 for the MoE models);
 * activations and outputs are IEEE binary16.  For x [M, K], packed weights of
 * W [N, K] and scales s [N, K/group]:
 *
 *     y[m, n] = sum_k x[m, k] * s[n, k / group] * q[n, k],   q in [-8, 7]
 *
 * accumulated in fp32 and rounded once to fp16 (round to nearest even).
 *
 * Storage (the reading this library fixes; the pages name only "int4 sym"):
 *   - code q is stored as the offset-binary nibble u = q + 8 (0..15);
 *   - eight nibbles per uint32 along K: element k = 8j + i of a row lives in
 *     bits [4i, 4i+4) of word j (low nibble first);
 *   - packed weights: uint32 [N, K/8] row-major (row n = output feature n);
 *   - scales: fp16 [N, K/group] row-major;
 *   - x: fp16 [M, K] row-major; y: fp16 [M, N] row-major;
 *   - MoE banks: packed uint32 [E, N, K/8], scales fp16 [E, N, K/group].
 * fp16 values cross the ABI as uint16_t bit patterns.
 *
 * Conventions for every entry point:
 *   - Every entry point that can fail returns a w4a16_status; nothing throws,
 *     aborts or prints.
 *   - Arguments are validated on the host before anything is launched; on a
 *     validation error no output is written.
 *   - m == 0, n == 0 or rows == 0 is a successful no-op.
 *   - The caller owns every buffer.  Device entry points take device pointers,
 *     run asynchronously on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise (w4a16_gemm_workspace_status, a
 *     diagnostic, is the one exception); host entry points take host pointers
 *     and are synchronous.
 *   - Alignment: x, y and packed weights 16-byte aligned, scales 2-byte
 *     aligned, offsets 4-byte aligned; K must be a multiple of `group`, and
 *     `group` must be 32 or 128 (the two sizes the pages name).
 *   - Calls on different streams may run concurrently; outputs must not alias
 *     inputs.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 2

/* The HIP stream type (hipStream_t is `struct ihipStream_t*`), declared here so
 * that C callers need not include the HIP headers. */
typedef struct ihipStream_t* w4a16_stream_t;

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL = 1,      /* a required pointer is NULL */
  W4A16_ERR_SHAPE = 2,     /* negative or inconsistent sizes, K % group != 0, M out of range */
  W4A16_ERR_GROUP = 3,     /* group size not in {32, 128} */
  W4A16_ERR_ALIGN = 4,     /* a pointer violates the alignment rules above */
  W4A16_ERR_WORKSPACE = 5, /* workspace missing or smaller than the query says */
  W4A16_ERR_HIP = 6,       /* the HIP runtime reported an error (launch or device query) */
  W4A16_ERR_RANGE = 7,     /* a value is out of range: a code outside [-8,7], a non-finite
                              weight, or a group scale that overflows fp16 */
  W4A16_ERR_TIMEOUT = 8    /* reported by w4a16_gemm_workspace_status only: a split-K fix-up of
                              an earlier w4a16_gemm gave up waiting for a partial tile */
} w4a16_status;

/* Version of this ABI (W4A16_ABI_VERSION). */
int w4a16_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* w4a16_status_str(int status);

/* ---------------------------------------------------------------- host ---- */

/*
 * Quantise fp32 weights w [n, k] (host) to packed codes (host, uint32 [n, k/8])
 * and fp16 scales (host, uint16 bits [n, k/group]).  Per group of `group`
 * consecutive k in a row: a = max |w| (fp32); s = fp16(a / 7) with the divide
 * in fp32 and round-to-nearest-even into fp16; q = clamp(rint(w / s), -8, 7)
 * with the divide in fp32 and ties to even; a group whose s is 0 gets q = 0.
 * Errors: NULL pointers, bad shapes/group, W4A16_ERR_RANGE for a non-finite w
 * or an s that overflows fp16 (nothing is written then).
 */
w4a16_status w4a16_quantize(const float* w, int64_t n, int64_t k, int32_t group,
                            uint32_t* packed, uint16_t* scales);

/*
 * Pack int8 codes q [n, k] (host, each in [-8, 7]) into uint32 [n, k/8] (host).
 * k must be a multiple of 8.  W4A16_ERR_RANGE if a code is out of range.
 */
w4a16_status w4a16_pack(const int8_t* q, int64_t n, int64_t k, uint32_t* packed);

/* Unpack uint32 [n, k/8] (host) back to int8 codes q [n, k] (host). */
w4a16_status w4a16_unpack(const uint32_t* packed, int64_t n, int64_t k, int8_t* q);

/* -------------------------------------------------------------- device ---- */

/*
 * Decode GEMV, 1 <= m <= 4 (the M = 1 decode step and the batched np4 decode
 * of the LLM170 CUDA/W4A16 page's benchmark tables): y = x . deq(W)^T.
 * All m rows share one pass over the packed weights.  x [m, k] and y [m, n]
 * fp16, packed [n, k/8], scales [n, k/group], all on the device.  Any k (a
 * multiple of group): up to w4a16_gemv_max_k(m, group) the activations are
 * staged in on-chip memory (LDS) whole; longer k runs on a kernel that stages
 * them in chunks, with the same result bars.  m > 4 is W4A16_ERR_SHAPE.
 */
w4a16_status w4a16_gemv(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                        uint16_t* y, int64_t m, int64_t n, int64_t k, int32_t group,
                        w4a16_stream_t stream);

/* Largest k for which w4a16_gemv stages the activations whole in LDS, for m
 * rows and this group size on the current device (0 if m is outside 1..4, the
 * group is invalid or no device is usable).  Informational: w4a16_gemv takes
 * longer k as well. */
int64_t w4a16_gemv_max_k(int64_t m, int32_t group);

/*
 * Bytes of device workspace w4a16_gemm needs for this problem on the current
 * device (0 means none; the pointer may then be NULL).  It is 0 for the
 * weight-streaming sizes (m <= 32 where those kernels run).  Returns 0 for
 * invalid shapes as well; w4a16_gemm reports those.  A workspace begins with a
 * 256-byte header holding the status word of w4a16_gemm_workspace_status.
 */
size_t w4a16_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t group);

/*
 * Prefill GEMM, any m >= 1 (the pp512 / pp4096 prefill of the same tables):
 * y = x . deq(W)^T with fp16 MFMA and fp32 accumulation.  Same layouts as
 * w4a16_gemv.  `workspace` (device, at least w4a16_gemm_workspace_bytes)
 * holds the partial tiles of the split-K schedule; the library leaves it in
 * the state it needs for the next call, so a buffer may be reused by calls
 * that run one after another on the same stream, but not by concurrent ones.
 * A fresh workspace must be zero-filled once before its first use.  For
 * m <= 32 the product is a weight stream and runs on weight-streaming kernels
 * (m <= 4: the decode GEMV kernels), with the same result bars; those need no
 * workspace (the query returns 0) and never touch one that is passed.
 * The split-K fix-up waits for other workgroups' partial tiles with a bounded
 * poll (about a second).  Should it ever give up (only if the device cannot
 * keep all of the launch's workgroups resident at once), the outputs of the
 * affected tiles are written as fp16 NaN, the call still returns W4A16_OK, and
 * the workspace's status word records it (w4a16_gemm_workspace_status).
 */
w4a16_status w4a16_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                        uint16_t* y, int64_t m, int64_t n, int64_t k, int32_t group,
                        void* workspace, size_t workspace_bytes, w4a16_stream_t stream);

/*
 * w4a16_gemm for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same product, the
 * same kernels and result bars, with no workspace argument.  The split-K
 * partial tiles go to a scratch array of the library itself (64 MiB + 3 KiB:
 * room for 256 persistent workgroups, one per CU of an MI355X), which each GPU
 * the library runs on holds from first use until the process ends.  Calls no
 * allocating routine.  A device whose plan needs more (more than 256 CUs)
 * gets W4A16_ERR_WORKSPACE.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (concurrent streams, or several host threads)
 * race and must not be issued; calls in order on one stream are fine.  Each
 * call clears the scratch's flags with a fill kernel before its product runs.
 * A split-K fix-up that gives up writes NaN, as in w4a16_gemm (its status
 * word is not readable here).
 */
w4a16_status w4a16_gemm_noalloc(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                uint16_t* y, int64_t m, int64_t n, int64_t k, int32_t group,
                                w4a16_stream_t stream);

/*
 * Diagnostic, not for the hot path: waits for the work queued on `stream`,
 * then reads the status word at the start of a w4a16_gemm workspace (device
 * pointer, at least 256 bytes).  Returns W4A16_ERR_TIMEOUT, and clears the
 * word, if a split-K fix-up of an earlier call on it gave up waiting (its
 * tiles were written as NaN); else W4A16_OK.  Synchronises the host.
 */
w4a16_status w4a16_gemm_workspace_status(void* workspace, size_t workspace_bytes, w4a16_stream_t stream);

/*
 * Fused gate/up projection of a SwiGLU feed-forward, 1 <= m <= 16 rows (the
 * SiLU-activated gate times the up projection: the rust-inference page's
 * "SwiGLU missing gate" item; gate and up fused in one pass as in the infr
 * page's Linear + GatedAct fusion).  packed [2n, k/8] and scales [2n, k/group]
 * hold 2n interleaved weight rows: row 2i is the gate row of output i, row
 * 2i + 1 its up row.  y [m, n] = fp16(SiLU(g) * u) with g, u the fp32-accumulated
 * products x . row^T and SiLU(g) = g / (1 + e^-g) in fp32; the 2 x m x n
 * intermediate never leaves the chip.  m <= 4 runs on the decode GEMV kernel
 * (each workgroup owns whole gate/up row pairs; no workspace), larger m on the
 * weight-streaming kernel.  Errors as w4a16_gemv (m > 16 is W4A16_ERR_SHAPE);
 * k == 0 writes zeros.
 */
w4a16_status w4a16_gemv_swiglu(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                               uint16_t* y, int64_t m, int64_t n, int64_t k, int32_t group,
                               w4a16_stream_t stream);

/*
 * MoE grouped GEMM (the routed-expert layers of the 35B-A3B MoE model on the
 * LLM170 CUDA/W4A16 page, g32).  x [rows, k] holds one row per (token, expert)
 * pair, sorted by expert; rows offsets[e] .. offsets[e+1]-1 belong to expert e
 * (offsets: device int32 [num_experts + 1], non-decreasing, offsets[0] = 0,
 * offsets[num_experts] = rows -- a precondition that is not checked, since
 * checking it would need a device-to-host copy).  packed [E, n, k/8] and
 * scales [E, n, k/group] hold the experts' weights.  y [rows, n]: row r is
 * x[r] . deq(W_e)^T for the expert e that owns row r.  No combine across
 * experts is done.
 */
w4a16_status w4a16_grouped_gemm(const uint16_t* x, const uint32_t* packed, const uint16_t* scales,
                                const int32_t* offsets, uint16_t* y, int32_t num_experts,
                                int64_t rows, int64_t n, int64_t k, int32_t group,
                                w4a16_stream_t stream);

/*
 * The routed-expert (MoE) steps either side of the grouped product, for the
 * 35B-A3B MoE layers of the LLM170 / infr pages (the MoE tiles and the batched
 * MoE path; the step around expert_gateup / expert_down).  All pointers are
 * device pointers; nothing synchronises.
 *
 * w4a16_moe_route: topk_ids int32 [tokens, topk] (expert of each (token, slot)
 * pair) -> offsets int32 [num_experts + 1] (rows of expert e are offsets[e] ..
 * offsets[e+1]-1), pair_token int32 [tokens * topk] (token of each grouped row)
 * and pair_row int32 [tokens, topk] (grouped row of each pair).  The order of
 * rows inside one expert is unspecified (it changes no product or combined
 * output).  An id outside [0, num_experts) gets pair_row = -1 and no row; then
 * offsets[num_experts] < tokens * topk.  1 <= num_experts <= 32768.
 */
w4a16_status w4a16_moe_route(const int32_t* topk_ids, int64_t tokens, int32_t topk, int32_t num_experts,
                             int32_t* offsets, int32_t* pair_token, int32_t* pair_row,
                             w4a16_stream_t stream);

/*
 * w4a16_grouped_gemm with the activations gathered: x [tokens, k] holds the
 * token rows unsorted and grouped row r reads x[pair_token[r]] (pair_token from
 * w4a16_moe_route), so no expert-sorted copy of x is made.  y [rows, n] as in
 * w4a16_grouped_gemm.  A pair_token outside [0, tokens) reads zeros.
 */
w4a16_status w4a16_grouped_gemm_gather(const uint16_t* x, const int32_t* pair_token, const uint32_t* packed,
                                       const uint16_t* scales, const int32_t* offsets, uint16_t* y,
                                       int32_t num_experts, int64_t rows, int64_t tokens, int64_t n,
                                       int64_t k, int32_t group, w4a16_stream_t stream);

/*
 * The experts' fused gate/up projection with its SwiGLU activation (the
 * expert_gateup role of the infr page's benchmarking section; the SwiGLU of the
 * rust-inference page; gate and up fused as the infr page's Linear + GatedAct):
 * packed [E, 2n, k/8] and scales [E, 2n, k/group] interleave each expert's gate
 * (even) and up (odd) weight rows; y [rows, n] row r = fp16(SiLU(g) * u) with
 * g, u the fp32-accumulated products of row r's activations with its expert's
 * gate and up rows, SiLU(g) = g / (1 + e^-g) in fp32.  With pair_token NULL, x
 * [rows, k] holds the rows sorted by expert (as for w4a16_grouped_gemm; tokens
 * is ignored); otherwise x [tokens, k] holds the token rows and grouped row r
 * reads x[pair_token[r]] (as for w4a16_grouped_gemm_gather).  offsets as for
 * w4a16_grouped_gemm.  The 2 x rows x n intermediate never leaves the chip.
 */
w4a16_status w4a16_grouped_gemm_swiglu(const uint16_t* x, const int32_t* pair_token, const uint32_t* packed,
                                       const uint16_t* scales, const int32_t* offsets, uint16_t* y,
                                       int32_t num_experts, int64_t rows, int64_t tokens, int64_t n, int64_t k,
                                       int32_t group, w4a16_stream_t stream);

/*
 * Router-weighted combine: out [tokens, n] fp16, out[t] = sum over slots j (in
 * order) of weights[t, j] * y_pairs[pair_row[t, j]], accumulated in fp32 and
 * rounded once.  y_pairs [rows, n] fp16 (the grouped product), weights fp32
 * [tokens, topk].  A pair_row outside [0, rows) contributes nothing.
 */
w4a16_status w4a16_moe_combine(const uint16_t* y_pairs, const int32_t* pair_row, const float* weights,
                               uint16_t* out, int64_t tokens, int32_t topk, int64_t rows, int64_t n,
                               w4a16_stream_t stream);

/* --------------------------------------------------------- measurement ---- */

/*
 * Streaming-read probe (measurement only, not part of the layer): reads the
 * `bytes` bytes at `buf` (device, 16-byte aligned, bytes a multiple of 1024)
 * once, with the decode GEMV's access pattern (one workgroup per CU, one
 * sequential stream of 1 KiB loads per wavefront), and stores one XOR of the
 * data per wavefront into `sink` (device uint32, at least
 * w4a16_hbm_read_probe_sink_words() words).  Its achieved bytes/time is the
 * same-box read bandwidth that the weight-streaming kernels are compared with,
 * beside the published HBM peak (the infr page, Validated models & performance,
 * gives decode GEMVs as a fraction of DRAM peak).
 */
w4a16_status w4a16_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                                  w4a16_stream_t stream);

/* Words of `sink` w4a16_hbm_read_probe needs on the current device (0: no device). */
int64_t w4a16_hbm_read_probe_sink_words(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
