/*
 * moe_q4.h - C ABI of the int4 expert-routed MoE layer library for AMD MI355X (gfx950).
 *
 * The library computes the prefill mixture-of-experts layer described on the
 * page "Perplexity Open Sources Lily: A Rust + Metal Inference Engine for
 * Qwen3.6-35B-A3B on Apple Silicon" (Technical Details: a router picks 8 of 256
 * experts plus one shared expert; groupwise affine 4-bit weights with 64
 * weights per group and FP32 accumulation, dequantised inside a grouped GEMM;
 * routing histogram, prefix scan, scatter and block map kept on the GPU with no
 * CPU synchronisation). Its Chinese section (技术解析, 预填充优化) adds that the
 * 64 weights of a group share one bfloat16 scale.
 *
 * Conventions shared by every entry point:
 *   - Plain C types only. "device" pointers point to GPU memory (hipMalloc or a
 *     torch CUDA tensor); "host" pointers point to CPU memory read during the call.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronises; scratch memory comes from the caller's workspace.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL means the
 *     default stream) and returns. Nothing is copied back to the host and no
 *     stream is synchronised inside a call.
 *   - Return value: MOE_OK or a negative moe_status. Arguments are validated
 *     before anything is launched; a call that fails validation launches
 *     nothing. A failed kernel launch returns MOE_ERR_HIP. The library never
 *     prints, aborts or throws.
 *   - Device-side contents (expert ids, offsets, tile maps) are trusted.
 *   - T == 0 is a no-op that returns MOE_OK once the sizes are valid.
 *   - Calls on different streams with different workspaces may run concurrently.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weights per quantisation group along the reduction dimension. */
#define MOE_Q4_GROUP 64
/* Rows per GEMM tile of moe_grouped_gemm_q4's tile maps, and the default tile
 * height of moe_layer_forward (dims.block_rows = 0). */
#define MOE_GEMM_BLOCK_ROWS 128
/* Bytes at the start of a moe_layer_forward workspace that hold state the
 * library keeps between layer calls (completion counters, the decode kernel's
 * epoch and its tagged hand-off words): zero before the first layer call, and
 * changed by nothing else afterwards (zeroing them again between calls is
 * allowed). */
#define MOE_WORKSPACE_HEAD_BYTES 190080
/* Byte offset, inside that head, of a uint32 status word: nonzero after a
 * decode-sized call whose persistent kernel, or whose one-launch routing
 * (T <= 8), gave up waiting (a bounded wait ran out, e.g. when other work kept
 * its workgroups from being resident); that call's outputs are then invalid.
 * It stays set until the head is zeroed. */
#define MOE_WORKSPACE_STATUS_OFFSET 16768
/* Largest supported expert count and top-k. */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 32

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    MOE_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    MOE_ERR_UNSUPPORTED = -5, /* valid request this build does not implement */
    MOE_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
} moe_status;

typedef enum {
    /* out[r][n] = sum_k A[src(r)][k] * W0_e[n][k], float32 [rows][N] */
    MOE_EPI_STORE_F32 = 0,
    /* out[r][n] = bf16(silu(A W0_e^T) * (A W1_e^T)), bf16 [rows][N] */
    MOE_EPI_SWIGLU_BF16 = 1
} moe_epilogue;

/* Host struct: sizes of one layer call.
 *   T tokens, H hidden size, I expert intermediate size, E routed experts,
 *   k experts chosen per token, block_rows rows per tile of the block map. */
typedef struct {
    int32_t T, H, I, E, k, block_rows;
} moe_dims;

/* Layouts of a moe_q4_weights stack. */
#define MOE_Q4_CANONICAL 0
#define MOE_Q4_PREPACKED 1

/* Host struct describing a stack of n_experts 4-bit matrices of shape [N][K]
 * (device pointers). The weight is W[n][k] = s[n][k/64] * q[n][k] + b[n][k/64]
 * with q the unsigned 4-bit code of element k of row n. G = K/64.
 * layout MOE_Q4_CANONICAL (0, the format every caller starts from):
 *   q : uint32 [n_experts][N][K/8]; nibble i (bits 4i..4i+3) of word w holds
 *       the code of element 8w+i of that row;
 *   s, b : bf16 [n_experts][N][G]; scale and bias of each run of 64
 *       consecutive elements along K.
 * layout MOE_Q4_PREPACKED (1, written by moe_prepack_q4; G even): the same
 * values reordered so that one group of consecutive rows is contiguous:
 *   q : uint32 [n_experts][G][N][8]: words 8g..8g+7 of row n at [g][n];
 *   s, b : uint32 [n_experts][G/2][N] (passed as uint16_t pointers): the bf16
 *       values of groups 2p (low half) and 2p+1 (high half) of row n at [p][n].
 * Every entry point accepts either layout; the two matrices of a gate/up pair
 * (gate and up, sh_gate and sh_up, W0 and W1) must share one. */
typedef struct {
    const uint32_t* q;
    const uint16_t* s;
    const uint16_t* b;
    int32_t n_experts, N, K;
    int32_t layout;
} moe_q4_weights;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* Workspace bytes moe_route or moe_layer_forward needs for these sizes
 * (0 when T == 0). Returns 0 for invalid sizes as well; call
 * moe_check_dims to tell the cases apart. */
size_t moe_workspace_bytes(const moe_dims* dims);

/* MOE_OK if the sizes are valid for moe_layer_forward, else the status it would return. */
int moe_check_dims(const moe_dims* dims);

/*
 * moe_route - top-k selection, softmax weights, and the routing tables
 * (histogram, exclusive prefix scan, stable scatter, block map) from fp32
 * router logits. Page "Perplexity Open Sources Lily ..." Technical Details
 * (router: 8 of 256 experts; GPU-resident routing histogram, prefix scan,
 * scatter and block map in one command buffer).
 *
 *   logits      device float [T][E] router logits (finite, or -inf with at
 *               least one finite value per token)
 *   logit_bias  device float [E] added to every row in fp32 first, or NULL
 *   dims        host; T >= 0, 1 <= k <= min(E, MOE_MAX_TOPK),
 *               E <= MOE_MAX_EXPERTS, block_rows >= 1 (H and I unused)
 *   topk_ids    device int32 [T][k]: the k largest (biased) logits of each
 *               token, in descending order, ties to the lower expert index
 *   topk_w      device float [T][k]: softmax over those k logits
 *   counts      device int32 [E]: pairs routed to each expert
 *   offsets     device int32 [E+1]: exclusive scan of counts; offsets[E] = T*k
 *   sorted_rows device int32 [T*k]: pair ids f = t*k + j grouped by expert,
 *               ascending f within an expert (a stable counting sort)
 *   row_of_pair device int32 [T*k]: inverse permutation, row_of_pair[sorted_rows[r]] = r
 *   tile_map    device int32 [moe_max_tiles(dims)][2]: (expert, first row) of each
 *               block_rows-row tile, experts ascending; entries past
 *               *num_tiles are left untouched
 *   num_tiles   device int32 [1]: number of valid tile_map entries
 *   workspace   device, at least moe_workspace_bytes(dims) bytes
 * The result is deterministic: repeated calls give identical bits.
 */
int moe_route(const float* logits, const float* logit_bias, const moe_dims* dims,
              int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* sorted_rows, int32_t* row_of_pair, int32_t* tile_map, int32_t* num_tiles,
              void* workspace, size_t workspace_bytes, void* stream);

/* Upper bound on the number of tiles moe_route can emit:
 * floor(T*k / block_rows) + min(E, T*k). */
int32_t moe_max_tiles(const moe_dims* dims);

/*
 * moe_grouped_gemm_q4 - grouped GEMM over expert-sorted row tiles with the
 * 4-bit weights dequantised inside the GEMM and FP32 accumulation (page
 * "Perplexity Open Sources Lily ..." Technical Details, prefill bullet; the
 * itinai.com post: weights are expanded only on chip, never as a full bf16
 * copy in memory).
 *
 * For every tile i < *num_tiles with (e, r0) = tile_map[i], every row r in
 * [r0, min(r0 + MOE_GEMM_BLOCK_ROWS, offsets[e+1])) is computed from the
 * activation row src(r) = sorted_rows ? sorted_rows[r] / row_div : r:
 *   MOE_EPI_STORE_F32   : out (float [.][N])   row r = A[src(r)] W0_e^T
 *   MOE_EPI_SWIGLU_BF16 : out (bf16  [.][N])   row r = bf16(silu(A[src] W0_e^T) * (A[src] W1_e^T))
 *     (silu(z) = z / (1 + exp(-z)); bf16 rounding is to nearest, ties to even)
 *
 *   A           device bf16 [a_rows][K]
 *   W0, W1      host structs; W1 only for SWIGLU (same n_experts, N, K as W0),
 *               K % 64 == 0 (else MOE_ERR_SHAPE) with an even number of 64-wide
 *               groups, K % 128 == 0 (else MOE_ERR_UNSUPPORTED: scale/bias words
 *               are read two groups at a time); N % 64 == 0 (SWIGLU) or
 *               N % 128 == 0 (STORE_F32); q, s and b 16-byte aligned
 *   a_rows      rows of A; a_rows * K * 2 must stay below 2^31 (A is addressed
 *               with 32-bit byte offsets), else MOE_ERR_UNSUPPORTED
 *   offsets, tile_map, num_tiles  device, as produced by moe_route with
 *               block_rows = MOE_GEMM_BLOCK_ROWS; max_tiles bounds *num_tiles
 *   workspace   device, at least moe_gemm_workspace_bytes(a_rows, K) bytes
 * Rows of `out` outside every tile are not written.
 */
int moe_grouped_gemm_q4(const uint16_t* A, int32_t a_rows, const int32_t* sorted_rows, int32_t row_div,
                        const moe_q4_weights* W0, const moe_q4_weights* W1,
                        const int32_t* offsets, const int32_t* tile_map, const int32_t* num_tiles,
                        int32_t max_tiles, int32_t epilogue, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

size_t moe_gemm_workspace_bytes(int32_t a_rows, int32_t K);

/*
 * moe_layer_forward - the whole MoE layer on one stream with no host
 * synchronisation between routing and the expert GEMMs:
 *   logits = fp32(x W_r^T) (+ logit_bias), top-k + softmax weights, routing
 *   tables, per routed row h = bf16(silu(x W_g^T) * (x W_u^T)), Y = h W_d^T,
 *   the shared expert on every token with weight 1, and
 *   y[t] = bf16(sum_j w[t][j] Y[row of (t, j)] + S[t]).
 * (Page "Perplexity Open Sources Lily ..." Technical Details, Model and prefill
 * bullets.) Calls with T <= 8 run decode-shaped kernels with the same result
 * (decode bullet: the chosen experts' weights are streamed once per step).
 * The call records no allocation or memset, so it may be captured in a HIP
 * graph on the caller's stream.
 *
 *   x            device bf16 [T][H]
 *   router_w     device bf16 [E][H]
 *   logit_bias   device float [E] or NULL
 *   gate, up     host structs, n_experts = E, N = I, K = H
 *   down         host struct,  n_experts = E, N = H, K = I
 *   sh_gate, sh_up, sh_down  the shared expert, n_experts = 1, same shapes
 *   dims         host; H % 64 == 0 and I % 64 == 0 (else MOE_ERR_SHAPE);
 *                an odd number of 64-wide groups in H or I returns
 *                MOE_ERR_UNSUPPORTED (the grouped GEMM reads scale/bias words
 *                two groups at a time); block_rows = 0 (MOE_GEMM_BLOCK_ROWS),
 *                32, 64 or 128 rows per routed tile (others:
 *                MOE_ERR_UNSUPPORTED); T*H*2, T*(k+1)*I*2 and E*H*2 bytes must
 *                stay below 2^31 (operands addressed with 32-bit byte offsets),
 *                else MOE_ERR_UNSUPPORTED
 *   y            device bf16 [T][H]
 *   logits_out   device float [T][E] or NULL: the logits routing used (biased)
 *   topk_ids_out device int32 [T][k] or NULL
 *   topk_w_out   device float [T][k] or NULL
 *   workspace    device, at least moe_workspace_bytes(dims) bytes. Its first
 *                MOE_WORKSPACE_HEAD_BYTES bytes hold state kept between calls
 *                (see MOE_WORKSPACE_HEAD_BYTES): allocate the workspace zeroed,
 *                and let nothing else write that head (moe_route never touches
 *                it; any other use of the buffer must zero it again before it
 *                serves a layer call). Calls that share a workspace must not
 *                run concurrently.
 */
int moe_layer_forward(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                      const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                      const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                      const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y,
                      float* logits_out, int32_t* topk_ids_out, float* topk_w_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Options of moe_layer_forward_ex (host struct; every field may be 0/NULL). */
typedef struct {
    /* device bf16 [H] or NULL. When given, the shared expert's output of token
     * t is scaled by g[t] = sigmoid(x[t] . shared_gate) (fp32 dot product and
     * logistic function), so y[t] = bf16(sum_j w[t][j] Y[t][j] + g[t] S[t]).
     * The pages name one shared expert beside the routed ones (page
     * "Perplexity Open Sources Lily ...", Technical Details, Model bullet) but
     * not how it is weighted; this gated form is an option, off by default.
     * 16-byte aligned. */
    const uint16_t* shared_gate;
    /* hipStream_t or NULL. When given, the shared expert's tiles (which need
     * no routing) run on this stream while the main stream routes; the main
     * stream waits for them before the combine. The page's single command
     * buffer and concurrent decode pass ("Perplexity Open Sources Lily ...",
     * Technical Details, prefill and decode bullets) in HIP stream form. The
     * side stream must be a different stream of the same device, at the
     * default priority. */
    void* side_stream;
    /* hipEvent_t handles created by the caller (no timing needed), required
     * with side_stream: fork_event is recorded on the main stream and waited
     * for on the side stream, join_event the other way round. */
    void* fork_event;
    void* join_event;
    /* Nonzero: calls with T <= 8, T * k <= 64, H == 2048 and I == 256 or 512
     * run the whole layer as one persistent launch (routing, gate/up and down
     * + combine as work items of one resident grid, handed over through
     * tagged words in the workspace head; see MOE_WORKSPACE_STATUS_OFFSET).
     * Zero (default): three launches. Same results up to the logits' summation
     * order at 5 <= T <= 8. Ignored with a side stream. */
    int32_t persistent_decode;
} moe_layer_options;

/*
 * moe_layer_forward_ex - moe_layer_forward with options (opts may be NULL,
 * which is moe_layer_forward). Same arguments, results and errors; in
 * addition MOE_ERR_ALIGN for a misaligned shared_gate and MOE_ERR_NULL for a
 * side stream without both events. The call may be captured in a HIP graph
 * on the main stream (the side stream forks from and joins back into it).
 */
int moe_layer_forward_ex(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                         const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                         const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                         const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y,
                         float* logits_out, int32_t* topk_ids_out, float* topk_w_out,
                         void* workspace, size_t workspace_bytes, void* stream,
                         const moe_layer_options* opts);

/* Number of stage boundaries moe_layer_forward_timed can mark. */
#define MOE_LAYER_STAGE_EVENTS 6

/*
 * moe_layer_forward_timed - moe_layer_forward that also records caller-created
 * HIP events (hipEvent_t handles passed as void*) on `stream` at its stage
 * boundaries, for measuring each kernel inside the timed region:
 *   events[0] before the activation prep kernel, [1] after it,
 *   [2] after the three routing kernels, [3] after the gate/up grouped GEMM,
 *   [4] after the down grouped GEMM, [5] after the combine kernel.
 * Only the first n_events (0..MOE_LAYER_STAGE_EVENTS) are recorded; every
 * recorded handle must be non-NULL (else MOE_ERR_NULL). Results are identical
 * to moe_layer_forward.
 */
int moe_layer_forward_timed(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                            const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                            const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                            const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y,
                            float* logits_out, int32_t* topk_ids_out, float* topk_w_out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events, int32_t n_events);

/* Bytes moe_prepack_q4 writes for a stack of these sizes (0 when K is not a
 * positive multiple of 128 or a size is not positive). */
size_t moe_prepack_q4_bytes(int32_t n_experts, int32_t N, int32_t K);

/*
 * moe_prepack_q4 - reorder a canonical stack into MOE_Q4_PREPACKED, done once
 * when the weights are loaded. The itinai.com post on the engine says the
 * 4-bit weights are expanded only on chip; the grouped GEMM reads one 64-wide
 * group of 32 consecutive rows per load, which in the canonical layout takes
 * 32 B from each of 32 lines and in the packed one whole lines.
 *   src     host struct, layout MOE_Q4_CANONICAL, K % 128 == 0 (an odd number
 *           of groups: MOE_ERR_UNSUPPORTED)
 *   dst     device, 16-byte aligned, at least moe_prepack_q4_bytes bytes;
 *           holds the codes, then the scale pairs, then the bias pairs
 *   packed  host struct filled on success: pointers into dst, same sizes,
 *           layout MOE_Q4_PREPACKED
 * Asynchronous on stream; src must stay valid until the work completes.
 */
int moe_prepack_q4(const moe_q4_weights* src, void* dst, size_t dst_bytes, moe_q4_weights* packed, void* stream);

/* Size of the device array behind moe_layer_forward_noalloc (per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * moe_layer_forward_noalloc - moe_layer_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without a workspace.
 * Its scratch memory is one MOE_NOALLOC_SCRATCH_BYTES device array per GPU,
 * part of the library's code object and held until the process ends; the call
 * makes no allocation of its own. The caller still passes every input and
 * output buffer.
 *   - Sizes whose workspace (moe_workspace_bytes) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_WORKSPACE and launch nothing:
 *     at H=2048, I=512, E=256, k=8 that is a few hundred tokens; decode-sized
 *     calls need well under 1 MiB.
 *   - The first call on a device resolves the array's address
 *     (hipGetSymbolAddress) and enqueues a kernel that zeroes its head; make
 *     that first call outside graph capture.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (other streams, other threads) race; serialise them.
 * Results are identical to moe_layer_forward's.
 */
int moe_layer_forward_noalloc(const uint16_t* x, const uint16_t* router_w, const float* logit_bias,
                              const moe_q4_weights* gate, const moe_q4_weights* up, const moe_q4_weights* down,
                              const moe_q4_weights* sh_gate, const moe_q4_weights* sh_up,
                              const moe_q4_weights* sh_down, const moe_dims* dims, uint16_t* y,
                              float* logits_out, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/*
 * moe_quantize_q4 - quantise bf16 weights into the layout the other entry
 * points read: for each row and each 64 consecutive elements along K, a bf16
 * scale s and bias b and 16-level codes q with W = s*q + b. The pages give the
 * format ("Perplexity Open Sources Lily ..." Technical Details, prefill bullet:
 * groupwise affine 4-bit, 64 weights per group; 技术解析: a bf16 scale per 64
 * weights) but not the quantiser; this one is min-max affine, each step in
 * fp32 (IEEE division, round half to even):
 *   lo = min, hi = max of the group (-0 taken as +0);
 *   s = bf16(fp32(hi - lo) / 15);  b = lo;
 *   q = 0 if s == 0, else min(15, max(0, rint((w - b) / s))).
 * Every weight is then reproduced within s/2, plus at most 15 * 2^-9 * s at
 * the top of a group from the bf16 rounding of s.
 *
 *   w      device bf16 [rows][K], 16-byte aligned, finite values
 *   rows   number of rows (for an expert stack: n_experts * N); 0 is a no-op
 *   K      multiple of 64
 *   q      device uint32 [rows][K/8], 16-byte aligned; element 8j+i of a row in
 *          bits 4i..4i+3 of word j
 *   s, b   device bf16 bit patterns [rows][K/64], 2-byte aligned
 * Returns MOE_OK, MOE_ERR_SHAPE (rows < 0, K not a positive multiple of 64,
 * rows*K above 2^40), MOE_ERR_NULL, MOE_ERR_ALIGN or MOE_ERR_HIP.
 */
int moe_quantize_q4(const uint16_t* w, int64_t rows, int32_t K, uint32_t* q, uint16_t* s, uint16_t* b,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
