/*
 * qmoe.h - C ABI of the MI355X (gfx950) quantized mixture-of-experts layer.
 *
 * The layer follows com.microsoft::QMoE semantics with SwiGLU experts, as the
 * onnxruntime pull-request pages describe them:
 *  - packed token-major I/O: x [T, hidden], router logits [T, num_experts],
 *    out [T, hidden]; sequences are concatenated without padding because
 *    routing is token-local ("Document and test packed token inputs for MoE and
 *    QMoE", Description);
 *  - raw router logits in; top-k, then a softmax over the k selected logits
 *    (same page, review comments on the CPU test harness and on top-k
 *    normalization);
 *  - integer experts with expert_weight_bits 4/3/2, block sizes 32/64/128,
 *    fp16 scales stored [N, K/block] and unsigned codes with a zero-point
 *    ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support", Description;
 *    "[CUDA/CPU] Add AVX2 INT4 cold-expert kernel and zero-cold doorbell
 *    short-circuit for QMoE offload", Motivation & Summary item 3: swiglu,
 *    fc1 rows = 2 * inter_size; "[CUDA] Add MoEPacked CPU/GPU hybrid offload
 *    and consolidate QMoE/GGUF offload optimizations", Summary: INT2 experts);
 *  - the routing-weighted combine accumulates in fp32 and rounds to the
 *    activation dtype once (the MoEPacked page, Key Changes item 4).
 *
 * Weight layout (device memory, owned by the caller, read-only here):
 *   fc1_codes  uint8  [E][2*inter][hidden*bits/8]  rows [0,I) gate, [I,2I) up
 *   fc1_scales fp16   [E][2*inter][hidden/block]
 *   fc2_codes  uint8  [E][hidden][inter*bits/8]
 *   fc2_scales fp16   [E][hidden][inter/block]
 * Codes are unsigned, K contiguous. INT4: two codes per byte, low nibble
 * first. INT2: four per byte, low bits first. INT3: eight codes per three
 * bytes, code i at bits [3i, 3i+3) of the little-endian 24-bit word.
 * W[n][k] = (q[n][k] - zero_point) * scale[n][k / block].
 *
 * Conventions for every call:
 *  - no exception crosses the ABI; each call returns a qmoe_status;
 *  - every argument is validated on the host before any device work; a call
 *    that returns an error has enqueued nothing;
 *  - device pointers must be 16-byte aligned;
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *    work is enqueued asynchronously and the call returns without
 *    synchronizing; only launch errors are reported (QMOE_ERR_HIP);
 *  - a handle may be used from one stream at a time (see qmoe_create);
 *  - environment variables read once, by qmoe_create, change nothing unless
 *    set: QMOE_FORCE_PATH=prefill|small|grouped|decode_split forces one
 *    path (grouped: the fused decode in groups of four up to 24 tokens;
 *    debugging, tests and measurement); QMOE_FUSED_GRID,
 *    QMOE_FUSED_EPOCH_START and QMOE_FUSED_SPIN_LIMIT are test hooks of the
 *    fused decode (a smaller grid, the epoch counter's start, the bound of
 *    its waits) that exist so the tests can reach its rare schedules and
 *    error paths.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qmoe_status {
    QMOE_OK = 0,
    QMOE_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad enum */
    QMOE_ERR_UNSUPPORTED = 2,   /* valid but not implemented (e.g. huge top_k) */
    QMOE_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    QMOE_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    QMOE_ERR_OOM = 5            /* host allocation failed */
} qmoe_status;

typedef enum qmoe_dtype {
    QMOE_F32 = 0,               /* x, logits and out are float32 */
    QMOE_BF16 = 1,              /* x, logits and out are bfloat16 */
    QMOE_F16 = 2                /* x, logits and out are float16 */
} qmoe_dtype;

/* qmoe_config.flags: FC1 rows stored interleaved, row 2n = gate n and row
 * 2n+1 = up n (scale rows in the same order), the exporter layout named in
 * the review of "[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support"
 * (producer/consumer contract). Without it rows [0, I) are the gate and rows
 * [I, 2I) the up projection. */
#define QMOE_FLAG_FC1_INTERLEAVED 1

/* Layer description, passed by value into qmoe_create and validated once. */
typedef struct qmoe_config {
    uint32_t struct_size;       /* sizeof(qmoe_config): ABI guard */
    int32_t top_k;              /* 1 <= top_k <= min(num_experts, 32) */
    int64_t hidden;             /* H > 0, multiple of block_size */
    int64_t inter;              /* I > 0, multiple of block_size */
    int64_t num_experts;        /* 1 <= E <= 1024 */
    int32_t bits;               /* 2, 3 or 4 */
    int32_t block_size;         /* 32, 64 or 128 */
    int32_t zero_point;         /* 0 <= zp < 2^bits, or -1 for 2^(bits-1) */
    int32_t act_dtype;          /* qmoe_dtype */
    int32_t normalize_routing;  /* 1: routing weights are the softmax over the k selected
                                   logits; 0: each selected expert's softmax probability
                                   over all num_experts logits (same top-k either way) */
    int32_t flags;              /* QMOE_FLAG_* bits; all others must be 0 */
    int64_t max_tokens;         /* largest T accepted by qmoe_forward (>= 0) */
} qmoe_config;

/* Device pointers to the expert weights (layout in the file comment). */
typedef struct qmoe_weights {
    const void *fc1_codes;
    const void *fc1_scales;
    const void *fc2_codes;
    const void *fc2_scales;
    /* Optional biases in the activation dtype, or NULL: fc1_bias [E, 2I] is
     * added to each FC1 row's output (gate and up rows, in their storage
     * order) before SwiGLU, fc2_bias [E, H] to the expert's output before the
     * routing-weighted combine ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU
     * offload support", commit notes). For T <= 4 such layers run the fused
     * decode (its instance that also loads biases and zero points) when
     * inter <= 768, else the split decode. */
    const void *fc1_bias;
    const void *fc2_bias;
    /* Optional zero-point tensors, or NULL: one unsigned code per row and
     * quant block (uint8 [E, 2I, H/bs] and [E, H, I/bs], laid out like the
     * scales) replacing the scalar zero_point, so W = (q - zp[n][k/bs]) * s.
     * For T <= 4 such layers run the fused decode when inter <= 768, else
     * the split decode. */
    const void *fc1_zero_points;
    const void *fc2_zero_points;
} qmoe_weights;

typedef struct qmoe_handle qmoe_handle;

/*
 * Create a layer handle. Validates the config and the weight pointers and
 * stores them; the weights are neither copied nor freed and must outlive the
 * handle. `device` is the HIP device ordinal the weights live on.
 * On success *out receives the handle; on error *out is set to NULL.
 *
 * Validation follows the pages' fail-closed admission: dimensions must be
 * positive and representable, the expert count nonzero, and enums in range
 * ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support", review-fix
 * commits on weights_prepacked normalization and E = 0 rejection).
 *
 * Besides host state, a handle whose layer the fused decode serves (bf16 or
 * fp16 activations, E <= 256, H <= 2048, I <= 1024) owns one device buffer
 * on `device`: the exchange area the fused decode's workgroups pass h and y
 * through, 256 + 4 * top_k * (inter + hidden) * 8 bytes (about 3 MB at the
 * Qwen3-30B-A3B shape), allocated and zeroed here and freed by
 * qmoe_destroy. Its entries carry a per-call epoch that the handle counts
 * on the host, so one handle must be used from one stream at a time: two
 * streams driving one handle concurrently race on that buffer. (Calls
 * under HIP graph capture never use it: see qmoe_forward.)
 * Errors: QMOE_ERR_INVALID_ARG for a bad config, pointer or device ordinal;
 * QMOE_ERR_UNSUPPORTED beyond this implementation's limits (E > 1024,
 * top_k > 32, hidden or inter > 8192); QMOE_ERR_HIP if a device call fails;
 * QMOE_ERR_OOM if the host allocation fails.
 */
qmoe_status qmoe_create(const qmoe_config *config, const qmoe_weights *weights, int device,
                        qmoe_handle **out);

/*
 * Bytes of device workspace qmoe_forward needs for `num_tokens` tokens
 * (0 <= num_tokens <= max_tokens). The workspace holds the routing arrays,
 * the expert-sorted permutation and tile list, the per-route intermediate
 * activations and the per-route fp32 FC2 outputs; it carries no state
 * between calls and needs no initialisation. The size is computed from the
 * shapes and checked by qmoe_forward, never assumed: a review on the pages
 * asks that the prefill scratch, computed by a workspace-size function, be
 * checked against every resolved device budget ("[CUDA] Add MoEPacked
 * CPU/GPU hybrid offload and consolidate QMoE/GGUF offload optimizations",
 * review comment on the device working budget).
 * Errors: QMOE_ERR_INVALID_ARG for a NULL handle or `bytes`, or num_tokens
 * outside [0, max_tokens].
 */
qmoe_status qmoe_workspace_size(const qmoe_handle *handle, int64_t num_tokens, size_t *bytes);

/*
 * The layer forward pass: out[t] = sum_j w[t][j] * FFN_{e[t][j]}(x[t]).
 *  x       device [num_tokens, hidden]       act_dtype, row-major
 *  logits  device [num_tokens, num_experts]  act_dtype, raw router logits
 *  out     device [num_tokens, hidden]       act_dtype (written)
 *  workspace / workspace_bytes: caller-owned device scratch of at least
 *          qmoe_workspace_size(num_tokens) bytes.
 * num_tokens == 0 returns QMOE_OK and launches nothing.
 *
 * The method: top-k of the raw router logits, softmax over the selected k,
 * the expert FFNs on dequantized weights W = (q - zp) * s with SwiGLU, and a
 * routing-weighted sum in fp32 rounded once ("Document and test packed token
 * inputs for MoE and QMoE", Description and review of the test harness;
 * "[CUDA/CPU] Add AVX2 INT4 cold-expert kernel and zero-cold doorbell
 * short-circuit for QMoE offload", Motivation & Summary item 3; "[CUDA] Add
 * MoEPacked CPU/GPU hybrid offload and consolidate QMoE/GGUF offload
 * optimizations", Key Changes item 4).
 *
 * Dispatch:
 *  - 1..4 tokens: the fused single-launch decode where it applies (see
 *    qmoe_create), else the split decode (three launches);
 *  - 5..8 tokens on layers the fused decode serves: the fused decode once
 *    per group of up to four tokens;
 *  - up to 256 tokens: routing, then the small-batch GEMMs (each active
 *    expert's weights streamed once per call into the fp16 matrix cores for
 *    up to 16 of its routes at a time), then the combine;
 *  - more tokens: routing, then the grouped fp16 matrix-core GEMMs over
 *    expert-sorted routes in tiles of 256, then the combine.
 * A call made while `stream` is being captured into a HIP graph takes the
 * split decode (1..4 tokens) or the batched paths (above): the fused
 * decode's per-call epoch cannot be replayed.
 *
 * The fused decode's workgroups exchange results through the handle's
 * buffer and each needs the others resident at once; its grid is one
 * workgroup per compute unit, so it assumes the device is otherwise idle
 * while it runs. A wait that runs out (a workgroup that could not start,
 * for instance) sets an error bit instead of hanging; outputs of the calls
 * since the last qmoe_decode_errors query may then be wrong, and that query
 * reports it.
 */
qmoe_status qmoe_forward(qmoe_handle *handle, const void *x, const void *logits, void *out,
                         int64_t num_tokens, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * Size in bytes of the device array qmoe_forward_noalloc uses as its
 * workspace (one array per GPU the library runs on, held until the process
 * ends).
 */
#define QMOE_NOALLOC_WORKSPACE_BYTES (32u << 20)

/*
 * qmoe_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, result and dispatch as qmoe_forward, without the workspace:
 * the call uses the library's own device array of
 * QMOE_NOALLOC_WORKSPACE_BYTES bytes on the handle's device and allocates
 * nothing. Calls whose workspace (qmoe_workspace_size) would exceed that size
 * return QMOE_ERR_WORKSPACE and enqueue nothing; at the Qwen3-30B-A3B layer
 * shape that allows every decode size and packed batches of about 400
 * tokens. Every handle on one GPU shares that GPU's array: calls on the same
 * GPU whose work overlaps in time (different streams, different threads)
 * race on it, and must be ordered by the caller. Nothing in it needs to
 * start at zero. QMOE_ERR_UNSUPPORTED for device ordinals of 64 and above.
 */
qmoe_status qmoe_forward_noalloc(qmoe_handle *handle, const void *x, const void *logits, void *out,
                                 int64_t num_tokens, void *stream);

/* Release a handle: its host state and, when it has one, its device
 * exchange buffer (after which no call may be in flight on it).
 * qmoe_destroy(NULL) returns QMOE_OK. */
qmoe_status qmoe_destroy(qmoe_handle *handle);

/* Static, human-readable text for a status code. */
const char *qmoe_status_string(int status);

/*
 * Test exports. Same conventions as above.
 *
 * qmoe_route runs only the routing stage of the batched paths on
 * `num_tokens` tokens (any count 1..max_tokens) and copies its results out:
 * the one-launch routing of the small-batch path when a forward of that
 * many tokens would take that path and its route list fits the launch, else
 * the chunked routing of the grouped GEMMs. The
 * expert-sorted route map with per-expert first offsets is the grouped
 * GEMMs' input ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support",
 * Description: sorted routes, tile descriptors, expert first-token offsets);
 * the order within an expert is the stable order of the route ids:
 *   topk_id        int32 [T, top_k]   selected experts, slot order
 *   topk_w         fp32  [T, top_k]   softmax over the selected logits
 *   expert_offsets int32 [E + 1]      exclusive prefix sum of routes per expert
 *   sorted_routes  int32 [T * top_k]  route ids r = t*top_k + j, stably sorted by expert
 *   inv_pos        int32 [T * top_k]  position of route r in sorted_routes
 * All output pointers are device pointers; any of them may be NULL to skip it.
 * Errors: QMOE_ERR_INVALID_ARG for a bad handle, count or logits pointer;
 * QMOE_ERR_WORKSPACE if the workspace is smaller than
 * qmoe_workspace_size(num_tokens).
 */
qmoe_status qmoe_route(qmoe_handle *handle, const void *logits, int64_t num_tokens,
                       int32_t *topk_id, float *topk_w, int32_t *expert_offsets,
                       int32_t *sorted_routes, int32_t *inv_pos, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * qmoe_dequant writes the dequantized matrix of one expert of FC1 (fc = 1,
 * [2*inter, hidden]) or FC2 (fc = 2, [hidden, inter]) using the kernels' own
 * routines, for W = (q - zp) * s ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU
 * offload support", Description: raw integer experts, block sizes
 * 32/64/128, scales [N, K/block]; "[CUDA/CPU] Add AVX2 INT4 cold-expert
 * kernel and zero-cold doorbell short-circuit for QMoE offload",
 * Motivation & Summary item 3: unsigned codes with a zero point):
 *   out_f32  device fp32 [N, K]: (q - zp) * s, exact, from the codes the
 *            decode paths' matrix operands carry (each code as bf16 128 + q)
 *   out_f16  device fp16 bits [N, K]: fp16((q - zp) * s), rounded once to
 *            nearest even, from the same routine the grouped GEMMs' staging
 *            calls
 * Either output may be NULL. Errors: QMOE_ERR_INVALID_ARG for a bad handle,
 * fc or expert.
 */
qmoe_status qmoe_dequant(qmoe_handle *handle, int fc, int64_t expert, float *out_f32,
                         uint16_t *out_f16, void *stream);

/*
 * Byte offsets, inside the workspace of a qmoe_forward call on `num_tokens`
 * tokens, of the routing results that call leaves behind: topk_id (int32
 * [T, top_k]) and topk_w (fp32 [T, top_k]), the top-k over raw logits and
 * the softmax over the selected ("Document and test packed token inputs for
 * MoE and QMoE", review of the test harness). Both paths write them.
 * Errors: QMOE_ERR_INVALID_ARG for a NULL argument or a count outside
 * [0, max_tokens].
 */
qmoe_status qmoe_workspace_routing(const qmoe_handle *handle, int64_t num_tokens,
                                   size_t *topk_id_offset, size_t *topk_w_offset);

/*
 * Error bits of the fused decode's bounded waits. A workgroup of the fused
 * decode that waits for another's FC1 result (h) or FC2 result (y) gives up
 * after a fixed number of polls, sets a bit and goes on, so a stalled
 * producer cannot hang the device. bit 0: an h wait ran out; bit 1: a y
 * wait ran out. Either means some output since the last query may be wrong.
 *
 * The bits accumulate over every qmoe_forward call on the handle since it
 * was created or last queried. This call waits for `stream` (the stream the
 * forward calls ran on; NULL = the null stream) to finish, copies the bits
 * to *bits and clears them: it is synchronous and meant for checks, not for
 * the hot loop. A handle whose layer never takes the fused decode reports 0.
 * Errors: QMOE_ERR_INVALID_ARG for a NULL handle or `bits`; QMOE_ERR_HIP if
 * the synchronisation or a copy fails (*bits is then 0).
 */
qmoe_status qmoe_decode_errors(qmoe_handle *handle, void *stream, uint32_t *bits);

/*
 * Profiling hook, for per-kernel time per layer as the pages measure it
 * ("[CUDA] Add INT4 and INT3 QMoE CPU/GPU offload support", GPU kernel time
 * per layer). When set, qmoe_forward calls fn(user, stage, name) on the
 * host right after it enqueues each kernel (stage = 1, 2, ... in launch order,
 * name = the kernel's role, a static string), and once with stage = 0 before
 * the first launch. It lets a caller record events on the stream between the
 * kernels of a real forward call. fn = NULL removes the hook. The hook must
 * not call back into the library.
 */
typedef void (*qmoe_stage_fn)(void *user, int stage, const char *name);
qmoe_status qmoe_set_stage_hook(qmoe_handle *handle, qmoe_stage_fn fn, void *user);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
