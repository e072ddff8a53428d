/*
 * moeq.h -- C ABI of libmoeq: the routed-expert MoE layer forward over 4-bit codebook
 * experts, hand-written HIP for gfx950 (MI355X).
 *
 * What the layer computes (sources are the pages' titles and sections):
 *   - geometry: "Round 7 -- Rewrite the GLM-5.2 routed-expert encoder", Ground truth /
 *     Model geometry: 256 routed experts, top-8, hidden 6144, moe_intermediate 2048;
 *   - expert: same brief, owner-locked decisions 4 and 6: I_e = silu(X Wg^T) * (X Wu^T),
 *     then the down contraction I_e Wd^T (K = 2048, N = 6144);
 *   - combine: README of GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "What had to be fixed" and
 *     "Shared residual rotations": expert outputs are router-weighted and summed per token;
 *   - weights: GLM-5.2-NF4-Lloyd-Experts-GPTQ model card, "Contents" (4-bit codes, two per
 *     byte with the even K index in the LOW nibble; one E8M0 scale byte per 32 consecutive K
 *     of a row) and "Codes are indices into the per-layer grid" (w = (-1)^(code>>3) *
 *     table[code & 7] * 2^(scale_byte - 127); the table is the layer's 8 fitted Lloyd-Max
 *     magnitudes, or per expert the E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}).
 *
 * Shapes: T tokens, H hidden, I expert intermediate, E experts, k experts per token.
 *   x        bf16 [T, H]                       (bf16 = uint16 bit patterns)
 *   logits   fp32 [T, E]
 *   gate/up  codes uint8 [E, I, H/2], scales uint8 [E, I, H/32]   (row n = output channel n)
 *   down     codes uint8 [E, H, I/2], scales uint8 [E, H, I/32]
 *   tables   fp32 [n_tables][8] HOST memory: 8 magnitudes per table
 *   table_id uint8 [E] device: which table each expert decodes with
 *
 * Conventions shared by every call:
 *   - All array pointers are DEVICE pointers owned by the caller, except `tables`, which is a
 *     host pointer read during the call (its values are copied into the kernel arguments).
 *   - The library never allocates, frees or synchronises. `stream` is a hipStream_t passed as
 *     void* (NULL = the null stream); every call only enqueues work on it.
 *   - Return value: MOEQ_OK, or a negative moeq_status; the arguments are checked before
 *     anything is launched, and on error nothing is launched. moeq_last_error() gives a
 *     thread-local message for the last failing call. Faults inside a kernel surface at the
 *     caller's next synchronisation, as for any HIP launch.
 *   - Results are deterministic: no floating-point atomics anywhere.
 *   - Size limits: 1 <= k <= E <= 256; H and I multiples of 64; T*k < 2^31.
 *   - Alignment: codes, x, inter and yp 16-byte aligned; scales 4-byte aligned.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moeq_status {
    MOEQ_OK = 0,
    MOEQ_EINVAL = -1,        /* invalid argument (null pointer, bad size, bad table value) */
    MOEQ_EUNSUPPORTED = -2,  /* valid but unsupported shape, alignment or mode */
    MOEQ_EWORKSPACE = -3,    /* workspace missing or too small */
    MOEQ_ELAUNCH = -4        /* a HIP launch reported an error */
};

/* Gate scoring. The pages say expert outputs are router-weighted but not how the weights are
 * formed, so two textbook forms are offered; both select the same k experts (the largest
 * logits: sigmoid is increasing).
 *   MOEQ_GATING_SOFTMAX_TOPK  softmax over the k selected logits
 *   MOEQ_GATING_SIGMOID_TOPK  sigmoid of each selected logit, divided by their sum (the
 *                             scoring of GLM-4.5-family routers, without the bias term and
 *                             group limit, which the pages do not mention) */
enum moeq_gating { MOEQ_GATING_SOFTMAX_TOPK = 0, MOEQ_GATING_SIGMOID_TOPK = 1 };

#define MOEQ_MAX_EXPERTS 256
/* At most 4 decode tables per call. Every workgroup of the projection kernels expands each
 * table into exact bf16 magnitudes for all 256 scale bytes (256 x 16 bytes = 4 KiB of LDS per
 * table) before it decodes; in the many-rows kernels the activation and code staging buffers
 * take 128 KiB of the CU's 160 KiB, which leaves room for 4 tables (16 KiB). The pages use two
 * per layer (the fitted grid and E2M1). */
#define MOEQ_MAX_TABLES 4

/* Position of intermediate channel c inside a row of `inter` (see moeq_gateup_swiglu):
 * within each aligned group of 8 channels the order is 0, 2, 4, 6, 1, 3, 5, 7. */
static inline int moeq_inter_slot(int c) {
    return (c & ~7) | (((c & 1) << 2) | ((c & 7) >> 1));
}

/* Thread-local message describing the last failing call of this thread ("" if none). */
const char* moeq_last_error(void);

/* Bytes of device workspace that moeq_gateup_swiglu and moeq_down need for these sizes
 * (0 means they accept ws = NULL). Currently 256 + T * H * 2 rounded up to 256: the first
 * 256 bytes hold the work-queue counters of the many-rows kernels (the call clears them on
 * its stream before use), the rest a copy of x that gate|up writes, when it takes the
 * many-rows kernels, with every 8-element group in the pair-split order of moeq_inter_slot
 * (the few-rows kernels reorder the rows they stage, in LDS). The workspace must be 16-byte
 * aligned;
 * its contents are scratch between calls (two calls that run at the same time need two
 * workspaces). */
size_t moeq_workspace_bytes(int T, int k, int E, int H, int I);

/*
 * Router logits: logits[t, e] = sum_h x[t, h] * router_w[e, h], products of bf16 values summed
 * in fp32 (GLM-5.2-EXL3-DENSE6-MTP78 model card, "Quant recipe": the router stays in BF16;
 * "Round 7" brief, "Target pipeline": the routing of a layer is its router applied to the
 * layer's activations). The summation order is fixed (the same bits on every call), not the
 * order of a sequential sum.
 *   x         bf16 [T, H]  in, row-major, 16-byte aligned
 *   router_w  bf16 [E, H]  in, row-major (one row per expert), 16-byte aligned
 *   logits    fp32 [T, E]  out, row-major, 4-byte aligned
 * T = 0 is a no-op. Errors: MOEQ_EINVAL for null pointers, T < 0, H <= 0, E outside [1, 256];
 * MOEQ_EUNSUPPORTED when H is not a multiple of 64, x or router_w is 2 GiB or more, or a
 * pointer is misaligned. The caller owns every buffer; nothing is allocated.
 */
int moeq_router_logits(const uint16_t* x, int T, int H, const uint16_t* router_w, int E,
                       float* logits, void* stream);

/*
 * Top-k routing. For each token t, topk_ids[t, 0..k) are the k experts with the largest
 * logits, in descending logit order under IEEE-754 totalOrder of the fp32 bit patterns;
 * equal bit patterns go to the lower expert id. topk_w[t, j] (fp32) is, for
 * MOEQ_GATING_SOFTMAX_TOPK, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected
 * logits, and for MOEQ_GATING_SIGMOID_TOPK, w_j = s_j / sum_i s_i with s = sigmoid(l),
 * evaluated so that no term overflows or all of them underflow. The gate values are finite
 * when the selected logits are. (Source for top-8 of 256: "Round 7" brief, Model geometry.)
 *   logits   fp32 [T, E]   in
 *   topk_ids int32 [T, k]  out
 *   topk_w   fp32 [T, k]   out
 * T = 0 is a no-op. Errors: MOEQ_EINVAL for null pointers, k < 1, k > E, E > 256, unknown
 * gating.
 */
int moeq_route_topk(const float* logits, int T, int E, int k, int gating, int32_t* topk_ids,
                    float* topk_w, void* stream);

/*
 * Group the T*k (token, slot) pairs by expert. Pair p = t*k + j with expert topk_ids[p].
 * Pairs are ordered by (expert, p) ascending -- a stable counting sort built from an expert
 * histogram and a wavefront prefix scan -- so the result is unique and deterministic.
 *   topk_ids       int32 [T*k]  in
 *   expert_offsets int32 [E+1]  out: rows of expert e are sorted positions
 *                               [expert_offsets[e], expert_offsets[e+1]); expert_offsets[E]
 *                               is the number of VALID pairs
 *   sorted_pair    int32 [T*k]  out: sorted position -> pair p
 *   pair_pos       int32 [T*k]  out: pair p -> sorted position
 * A pair whose id lies outside [0, E) is not dropped silently: it is placed after every valid
 * pair (positions >= expert_offsets[E], in p order), no expert computes it, and
 * moeq_unpermute_combine writes NaN for its token. Callers detect it as expert_offsets[E] <
 * T*k. Errors: MOEQ_EINVAL for null pointers or sizes out of range.
 */
int moeq_permute_by_expert(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                           int32_t* sorted_pair, int32_t* pair_pos, void* stream);

/*
 * moeq_route_topk followed by moeq_permute_by_expert, with the same results and the same
 * arguments (the logits in, the five routing arrays out). Up to 64 tokens it is one launch (one
 * workgroup routes and then permutes); beyond, it launches the two kernels. Errors: the union
 * of the two calls' errors. (Few-token decode steps spend a launch less on the front of the
 * path; the pages' decode kernels favour fewer launches: README of
 * GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Tuning" / "Why".)
 */
int moeq_route_permute(const float* logits, int T, int E, int k, int gating, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair,
                       int32_t* pair_pos, void* stream);

/*
 * Fused gate|up projection and SwiGLU ("Round 7" brief, decision 4), with the weights decoded
 * from 4-bit codes as they are streamed (model card, "Codes are indices into the per-layer
 * grid"). For each sorted row r of expert e (pair p = sorted_pair[r], token t = p / k):
 *     g = X[t] . Wg[e][n],  u = X[t] . Wu[e][n]          (fp32 accumulation)
 *     inter[r][moeq_inter_slot(n)] = bf16(silu(g) * u)   (round to nearest even)
 * Each weight is decoded exactly: bf16(sign * table[table_id[e]][code & 7] * 2^(s - 127)),
 * one round-to-nearest-even of the exact product (s = 255 decodes to NaN).
 *   x        bf16 [T, H]
 *   expert_offsets, sorted_pair: from moeq_permute_by_expert
 *   gate/up codes uint8 [E, I, H/2], scales uint8 [E, I, H/32]
 *   tables   HOST fp32 [n_tables][8], 1 <= n_tables <= MOEQ_MAX_TABLES; every entry must be
 *            finite and non-negative with a clear sign bit (they are magnitudes)
 *   table_id uint8 [E]; an expert whose id is >= n_tables writes NaN rows (never a guess)
 *   inter    bf16 [T*k, I] out, rows by sorted position, channels in moeq_inter_slot order;
 *            only rows < expert_offsets[E] are written. It is the library's layout for the
 *            intermediate, read back by moeq_down.
 *   ws       device workspace of at least moeq_workspace_bytes(T, k, E, H, I) bytes
 * T = 0 is a no-op once the sizes and tables pass (the arrays may then be NULL).
 * Errors: MOEQ_EINVAL (null pointer, sizes, table values), MOEQ_EUNSUPPORTED (H or I not a
 * multiple of 64, misalignment), MOEQ_EWORKSPACE.
 */
int moeq_gateup_swiglu(const uint16_t* x, int T, int H, int I, int E, int k,
                       const int32_t* expert_offsets, const int32_t* sorted_pair,
                       const uint8_t* gate_codes, const uint8_t* gate_scales,
                       const uint8_t* up_codes, const uint8_t* up_scales, const float* tables,
                       int n_tables, const uint8_t* table_id, uint16_t* inter, void* ws,
                       size_t ws_bytes, void* stream);

/* Length of the library's static scratch array: the most scratch moeq_gateup_swiglu_static
 * can use. 32 MiB + 256 bytes covers moeq_workspace_bytes for T * H <= 16,777,216, e.g. up to
 * 2730 tokens at H = 6144. */
#define MOEQ_STATIC_SCRATCH_BYTES (((size_t)32 << 20) + 256)

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): moeq_gateup_swiglu without the workspace
 * arguments. Its scratch (moeq_workspace_bytes(T, k, E, H, I) bytes: the work-queue counters
 * and the pair-split copy of x of the many-rows kernels) lives in a static device array of
 * this library,
 * MOEQ_STATIC_SCRATCH_BYTES long, which every GPU the library runs on holds until the process
 * ends. The call allocates nothing; its first call on a device looks that array's address up
 * on the device. Arguments, kernels and results are those of moeq_gateup_swiglu.
 * Calls that overlap on one GPU (other streams, other threads) share the array and race:
 * serialise them. Each call clears what must start at zero itself (on its stream).
 * Errors: as moeq_gateup_swiglu; MOEQ_EWORKSPACE, with nothing launched, when the call needs
 * more than MOEQ_STATIC_SCRATCH_BYTES; MOEQ_ELAUNCH when the array's address cannot be found.
 */
int moeq_gateup_swiglu_static(const uint16_t* x, int T, int H, int I, int E, int k,
                              const int32_t* expert_offsets, const int32_t* sorted_pair,
                              const uint8_t* gate_codes, const uint8_t* gate_scales,
                              const uint8_t* up_codes, const uint8_t* up_scales,
                              const float* tables, int n_tables, const uint8_t* table_id,
                              uint16_t* inter, void* stream);

/*
 * Down projection with the gate weight applied ("Round 7" brief, decision 6; README of
 * GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "What had to be fixed": router weighting happens in the
 * down epilogue). For each sorted row r of expert e, pair p = sorted_pair[r]:
 *     yp[r][h] = topk_w[p] * (inter[r] . Wd[e][h])       (fp32 accumulation)
 *   inter  bf16 [T*k, I] from moeq_gateup_swiglu
 *   topk_w fp32 [T*k] from moeq_route_topk
 *   down codes uint8 [E, H, I/2], scales uint8 [E, H, I/32]
 *   yp     fp32 [T*k, H] out; rows >= expert_offsets[E] are not written
 * Tables, table_id, ws, T = 0 and errors as for moeq_gateup_swiglu.
 */
int moeq_down(const uint16_t* inter, int T, int H, int I, int E, int k,
              const int32_t* expert_offsets, const int32_t* sorted_pair, const float* topk_w,
              const uint8_t* down_codes, const uint8_t* down_scales, const float* tables,
              int n_tables, const uint8_t* table_id, float* yp, void* ws, size_t ws_bytes,
              void* stream);

/*
 * Sum each token's k expert rows back into the residual space (README of
 * GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Shared residual rotations": routing-weighted and summed
 * back). In fp32, slots in fixed order j = 0..k-1:
 *     y[t] = bf16( sum_j yp[pair_pos[t*k + j]]  (+ residual[t]) )
 *   yp        fp32 [T*k, H] from moeq_down (gate weights already applied)
 *   pair_pos, expert_offsets: from moeq_permute_by_expert (a pair at a position >=
 *             expert_offsets[E] had an invalid expert id: its token's row becomes NaN)
 *   residual  bf16 [T, H] or NULL
 *   y         bf16 [T, H] out; may be the same buffer as residual (in-place update)
 * Errors: MOEQ_EINVAL for null pointers or bad sizes.
 */
int moeq_unpermute_combine(const float* yp, const int32_t* pair_pos, const int32_t* expert_offsets,
                           int T, int k, int E, int H, const uint16_t* residual, uint16_t* y,
                           void* stream);

/*
 * The shared expert (README of GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Checkpoint layout update
 * (2026-08-10): BF16 shared experts, merged online K6" and "What changed and why": each routed
 * layer also carries one shared gate/up/down MLP, 3 x 6144 x 2048 weights, with gate and up
 * merged into one launch). Stored here in the routed experts' 4-bit format and run on every
 * token with weight 1 by the same projection kernels, gate|up merged:
 *     inter[t][moeq_inter_slot(n)] = bf16(silu(X[t] . Wg[n]) * (X[t] . Wu[n]))
 *     z[t] = inter[t] . Wd^T                           (fp32)
 *   x        bf16 [T, H]
 *   gate/up codes uint8 [I, H/2], scales uint8 [I, H/32]; down codes uint8 [H, I/2], scales
 *            uint8 [H, I/32] (one expert of the routed layout)
 *   tables   HOST fp32 [n_tables][8] as for the routed projections; table_id uint8 [1] on the
 *            device (an id >= n_tables writes NaN rows)
 *   inter    bf16 [T, I] out (row t = token t)
 *   z        fp32 [T, H] out, for moeq_unpermute_combine_shared
 *   ws       moeq_shared_workspace_bytes(T, H, I) bytes, 256-byte aligned: the identity
 *            routing of the call (offsets, rows, unit gate weights) and the projections'
 *            workspace. Scratch between calls; calls that run at the same time (the shared
 *            expert on its own stream beside the routed path, say) need their own.
 * Sizes and alignment as for moeq_gateup_swiglu / moeq_down with E = 1, k = 1. T = 0 is a
 * no-op. Errors: MOEQ_EINVAL for null pointers or bad sizes, MOEQ_EUNSUPPORTED for shapes or
 * alignment, MOEQ_EWORKSPACE for a missing or short workspace; both projections are validated
 * before anything is launched.
 */
size_t moeq_shared_workspace_bytes(int T, int H, int I);
int moeq_shared_expert(const uint16_t* x, int T, int H, int I, const uint8_t* gate_codes,
                       const uint8_t* gate_scales, const uint8_t* up_codes,
                       const uint8_t* up_scales, const uint8_t* down_codes,
                       const uint8_t* down_scales, const float* tables, int n_tables,
                       const uint8_t* table_id, uint16_t* inter, float* z, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moeq_unpermute_combine with the shared expert's output added after the routed slots and
 * before the residual, all in fp32 (the same README, "Checkpoint layout update"):
 *     y[t] = bf16( sum_j yp[pair_pos[t*k + j]] + shared_z[t]  (+ residual[t]) )
 *   shared_z fp32 [T, H] from moeq_shared_expert, 16-byte aligned, or NULL (then the call is
 *            moeq_unpermute_combine)
 * Other arguments and errors as for moeq_unpermute_combine.
 */
int moeq_unpermute_combine_shared(const float* yp, const int32_t* pair_pos,
                                  const int32_t* expert_offsets, int T, int k, int E, int H,
                                  const float* shared_z, const uint16_t* residual, uint16_t* y,
                                  void* stream);

/*
 * The whole few-rows (decode) layer in one cooperative launch: moeq_route_topk,
 * moeq_permute_by_expert, moeq_gateup_swiglu, moeq_down and moeq_unpermute_combine with the
 * same results, run as phases of one grid separated by grid barriers (README of
 * GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Tuning" / "Why": one fused launch per layer, a grid the
 * size of the machine; cutting launches gained decode throughput). Workgroup 0 routes and
 * permutes while the others fill their decode tables; then gate|up, down and the combine run
 * on the whole grid. The projections' outputs are written with device-coherent stores, so the
 * barriers between the phases need no cache write-back or invalidation.
 *   x, logits, weights, tables, table_id, gating: as for the per-step calls
 *   residual bf16 [T, H] or NULL; y bf16 [T, H] out (may be the residual buffer)
 *   ws       moeq_moe_decode_workspace_bytes(T, k, E, H, I) bytes, 256-byte aligned: the
 *            barrier words, routing arrays, intermediate and expert outputs
 *            (scratch between calls; calls that overlap need their own). Bytes 8..47 receive
 *            five 64-bit stamps of the device's constant 100 MHz clock, taken by workgroup 0
 *            at the start and after each of the four phases (for profiling).
 * Requires T * k <= 4096 (the few-rows kernels' limit). A grid barrier that waits more than
 * about a second gives up instead of hanging and marks the call: moeq_moe_decode_check
 * synchronizes the stream and reports it (MOEQ_ELAUNCH), as it reports nothing otherwise.
 * Errors: as for the per-step calls; MOEQ_EUNSUPPORTED above 4096 rows; MOEQ_ELAUNCH when the
 * device refuses the cooperative launch.
 */
size_t moeq_moe_decode_workspace_bytes(int T, int k, int E, int H, int I);
int moeq_moe_decode(const uint16_t* x, const float* logits, int T, int H, int I, int E, int k,
                    int gating, const uint8_t* gate_codes, const uint8_t* gate_scales,
                    const uint8_t* up_codes, const uint8_t* up_scales, const uint8_t* down_codes,
                    const uint8_t* down_scales, const float* tables, int n_tables,
                    const uint8_t* table_id, const uint16_t* residual, uint16_t* y, void* ws,
                    size_t ws_bytes, void* stream);
int moeq_moe_decode_check(const void* ws, void* stream);

/*
 * Encode bf16 expert weights into the 4-bit format (GLM-5.2-NF4-Lloyd-Experts-GPTQ model card,
 * "Codes are indices into the per-layer grid": the grid holds absolute magnitudes and each
 * block of 32 weights along K has a power-of-two scale, stored as the byte e + 127; "Contents":
 * two codes per byte, the even K in the low nibble). Per block: e is the smallest integer with
 * table[7] * 2^e >= max |w| (clamped to [-127, 127]; an all-zero block gets byte 0, a block
 * holding an Inf or NaN gets byte 255 and zero codes); per weight: bits 0..2 index the
 * magnitude nearest to |w| / 2^e (ties to the lower index; decided exactly), bit 3 is set for
 * w < 0 (not for -0).
 *   w        bf16 [E, N, K] device, 16-byte aligned, K a multiple of 32
 *   tables   HOST fp32 [n_tables][8], 1 <= n_tables <= MOEQ_MAX_TABLES: finite magnitudes,
 *            non-decreasing, table[7] > 0
 *   table_id uint8 [E] device: the table of each expert (an id >= n_tables encodes NaN blocks)
 *   codes    uint8 [E, N, K/2] out, 16-byte aligned, or NULL
 *   scales   uint8 [E, N, K/32] out, or NULL
 *   row_err  fp64 [E * N] out, 8-byte aligned, or NULL: per row, sum over K of
 *            (w - bf16 dequantisation)^2 in fp64 (NaN when a block has byte 255)
 * Errors: MOEQ_EINVAL for bad sizes, null pointers or tables; MOEQ_EUNSUPPORTED for K not a
 * multiple of 32 or misalignment. Nothing is allocated.
 */
int moeq_quantize(const uint16_t* w, int E, int N, int K, const float* tables, int n_tables,
                  const uint8_t* table_id, uint8_t* codes, uint8_t* scales, double* row_err,
                  void* stream);

/*
 * One step of the weighted Lloyd-Max grid fit (the model card, "What this is": 8 magnitudes
 * per layer fitted over the pooled ratios |W / 2^e| of all experts' gate, up and down weights,
 * each ratio weighted by (2^e)^2). Over the bf16 weights [E, N, K]: e per block for the top
 * magnitude gmax (the moeq_quantize rule), each ratio r = |w| / 2^e assigned to its nearest
 * entry of `table` (ties to the lower), and per entry m the fp64 sums
 *     stats[m] = sum (2^e)^2 r,  stats[8 + m] = sum (2^e)^2,  stats[16 + m] = sum (2^e)^2 (r - table[m])^2
 * Blocks holding an Inf or NaN are skipped. The next table is stats[m] / stats[8 + m] (keep
 * table[m] where the sum of weights is 0). With accumulate != 0 the sums are added to stats
 * (pooling several calls, in call order), else they overwrite it. Summation order is fixed.
 *   table  HOST fp32 [8], finite, non-decreasing, table[7] > 0; gmax > 0 finite
 *   stats  fp64 [24] device
 *   ws     moeq_lloyd_workspace_bytes(E, N) bytes, 8-byte aligned (per-workgroup partial sums)
 * Errors as for moeq_quantize; MOEQ_EWORKSPACE for a missing or short workspace.
 */
size_t moeq_lloyd_workspace_bytes(int E, int N);
int moeq_lloyd_stats(const uint16_t* w, int E, int N, int K, const float* table, float gmax,
                     int accumulate, double* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * One Lloyd-Max update from the sums of moeq_lloyd_stats (GLM-5.2-NF4-Lloyd-Experts-GPTQ model
 * card, "What this is": the grid is a weighted Lloyd-Max fit). HOST arrays: stats [24] as
 * moeq_lloyd_stats leaves them (copied to the host by the caller), table [8] the magnitudes
 * the sums were taken against, next [8] out: magnitude m moves to the weighted mean of its
 * ratios, next[m] = fp32(stats[m] / stats[8 + m]) (fp64 quotient, one rounding to nearest),
 * or keeps table[m] when no ratio fell to it (stats[8 + m] = 0). sq_error (may be NULL) gets
 * the weighted squared error of the assignment the sums describe, the sum of stats[16..23]
 * in index order. next may equal table. Runs on the host; no device work. Errors:
 * MOEQ_EINVAL for null stats, table or next.
 */
int moeq_lloyd_update(const double* stats, const float* table, float* next, double* sq_error);

/*
 * Per-expert choice between two encodings (the model card, "Provenance": each expert's winner
 * is chosen against an E2M1 control arm): err_a, err_b fp64 [E * N] row errors of one matrix
 * of every expert from moeq_quantize under two tables. Per expert the two sums over its N rows
 * (row order) are written to expert_err [2E] (a, b), or added to it with accumulate != 0 (the
 * gate, up and down matrices of the experts in three calls); table_id[e] = 1 when the second
 * total is strictly smaller, else 0. expert_err may be NULL only without accumulate.
 * Errors: MOEQ_EINVAL for bad sizes or null pointers.
 */
int moeq_select_arms(const double* err_a, const double* err_b, int E, int N, int accumulate,
                     uint8_t* table_id, double* expert_err, void* stream);

/*
 * Test entry point: decode whole matrices with the same device decode path the two
 * projections use (model card, "Codes are indices into the per-layer grid").
 *   codes uint8 [E, N, K/2], scales uint8 [E, N, K/32], out bf16 [E, N, K] (natural K order)
 * K must be a multiple of 64. Tables and table_id as above.
 */
int moeq_debug_dequant(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                       const float* tables, int n_tables, const uint8_t* table_id, uint16_t* out,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEQ_H */
