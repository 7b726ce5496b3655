/*
 * tsoftmax: temperature softmax over an LLM vocabulary, and inverse-CDF token
 * draws, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the pull-request page "fix(kernel): avoid nan in
 * triton sampling softmax when a chunk starts with -inf" (FreeToken pull
 * request 654).
 *  - Test paragraph: every row b of the logits is divided by its own
 *    temperature t[b] and normalised with a softmax over the vocabulary.
 *  - Bug and fix paragraphs: masked logits are -inf; a column chunk whose
 *    first block is all -inf must add nothing to its row (shift by 0 while the
 *    running max is still -inf) instead of turning the row into NaN, and a
 *    fully masked chunk contributes 0 to the row's rescaled sum.
 *  - Scope paragraph and the sampling row of the results table: the
 *    probabilities feed a draw of token ids that must always land on an
 *    allowed (finite-logit) id.
 *
 * All entry points are C functions on plain pointers and sizes. Every array
 * is owned by the caller and lives in device memory of the current HIP device
 * (except where a pointer is documented as host memory). Calls are
 * asynchronous on `stream` (NULL = the default stream): they enqueue kernels
 * and return without synchronising or reading device memory on the host.
 * Calls on one stream are ordered; calls on different streams may run
 * concurrently and each stream gets its own small workspace.
 *
 * Thread safety: all functions may be called from several host threads.
 */
#ifndef TSOFTMAX_H_
#define TSOFTMAX_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSOFTMAX_ABI_VERSION 1

typedef enum ts_status {
    TS_OK = 0,
    /* A pointer, size or alias rule below was broken. Nothing was launched. */
    TS_ERR_INVALID_ARGUMENT = 1,
    /* The HIP runtime reported an error (launch or query). */
    TS_ERR_HIP = 2,
    /* The library could not allocate its workspace. */
    TS_ERR_OUT_OF_MEMORY = 3,
    /* The stream is being captured into a graph and the call needs a larger
     * workspace than ts_reserve() set aside for it; no allocation is made
     * during capture. Nothing was launched. */
    TS_ERR_NOT_RESERVED = 4,
    /* A fused kernel's bounded wait for the other chunks of its row ran out
     * (reported by ts_device_errors only): something else on the device kept
     * some of the row's workgroups from running. The waiting workgroup then
     * formed the missing chunk partials from the logits itself, bit for bit
     * as their own workgroups form them, so the results are exact; the code
     * reports the slow path. */
    TS_ERR_SYNC_TIMEOUT = 5
} ts_status;

/* How ts_softmax_variant splits the work. Defined by: the pull-request page,
 * bug paragraph (one program per row and column chunk computing a running max
 * and sum, then a finalize that combines the chunks with a global rescale).
 *   TS_VARIANT_AUTO    - pick from (B, V) with the built-in table (ts_plan).
 *   TS_VARIANT_SPLIT   - two kernels: per-chunk (max, scaled sum) partials,
 *                        then a finalize fused into the write of the probs.
 *                        Reads the logits twice.
 *   TS_VARIANT_ROWWISE - one workgroup per row, no partials. Reads the logits
 *                        once when the row fits in the workgroup's registers,
 *                        else twice.
 *   TS_VARIANT_FUSED   - one kernel: each workgroup keeps its chunk in
 *                        registers while the per-chunk partials are exchanged
 *                        through tagged per-row slots in the stream's
 *                        workspace, then writes the probs. Reads the logits
 *                        once. Rows of at most 256 chunks. Its grid is sized
 *                        to what the device holds at once; should the device be
 *                        shared with work that keeps some of a row's
 *                        workgroups from running, a row's wait can run out:
 *                        the waiting workgroup then forms the missing partials
 *                        itself (exact result, reported as TS_ERR_SYNC_TIMEOUT
 *                        by ts_device_errors). SPLIT and ROWWISE never wait. */
typedef enum ts_variant {
    TS_VARIANT_AUTO = 0,
    TS_VARIANT_SPLIT = 1,
    TS_VARIANT_ROWWISE = 2,
    TS_VARIANT_FUSED = 3
} ts_variant;

/*
 * probs[b, :] = softmax(logits[b, :] / temps[b]) for b in [0, B).
 *
 * Defined by: the pull-request page, test paragraph (each row divided by its
 * own temperature, then a softmax over the vocabulary, checked against
 * torch.softmax) and fix paragraph (a column chunk whose leading block is all
 * -inf adds nothing; a fully masked chunk contributes 0 to the rescaled sum,
 * so the row stays finite while it keeps a finite logit).
 *
 * logits : [B, V] float32, row-major, contiguous (row pitch V elements).
 *          Entries are finite or -inf (masked). Each row must keep at least
 *          one finite entry; a row of only -inf gives unspecified output.
 * temps  : [B] float32, every value finite and > 0 (not checked: checking
 *          would need a device read).
 * out    : [B, V] float32, row-major, contiguous. out == logits (exact
 *          alias, in place) is allowed; any other overlap of out with logits
 *          or temps is rejected.
 * Result : for a row with at least one finite logit every output is finite,
 *          a -inf logit gives exactly 0, and the row sums to 1 within float32
 *          rounding. No alignment beyond float's 4 bytes is required: rows
 *          are read and written 16 bytes at a time either way (aligned when
 *          logits and out are 16-byte aligned and V % 4 == 0, unaligned
 *          otherwise, the row's last partial float4 element by element).
 * Errors : TS_ERR_INVALID_ARGUMENT for B < 0, V < 1, V > INT32_MAX,
 *          B*V*4 not addressable, a NULL pointer when B > 0, or an illegal
 *          overlap. B == 0 is a no-op returning TS_OK.
 *          TS_ERR_NOT_RESERVED, TS_ERR_OUT_OF_MEMORY, TS_ERR_HIP as above.
 */
ts_status ts_softmax(const float* logits, const float* temps, int64_t B, int64_t V,
                     float* out, hipStream_t stream);

/*
 * ts_softmax for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, work split, kernels and result (bit for bit) as ts_softmax, but
 * it never allocates: instead of the per-stream workspace it uses one
 * 4 MiB + 256 B device array that the library holds on each GPU until the
 * process ends (fused-kernel slots for up to 1024 rows, split partials for up
 * to 262144 (row, chunk) pairs). Every call on a GPU shares that GPU's array
 * whatever its stream, so calls that overlap on one GPU race: keep them on one
 * stream, or otherwise ordered. The array needs no clearing between calls.
 * Its bounded-wait flag is not reported (ts_device_errors covers the
 * workspaces only); a wait that runs out still gives the exact result.
 * Errors : as ts_softmax, plus TS_ERR_INVALID_ARGUMENT when the call's work
 *          split needs more than the array holds: the fused split with more
 *          than 1024 rows, or the split pair with more than 262144 - B
 *          (row, chunk) pairs. Calls that take the one-workgroup-per-row
 *          kernel need no scratch and have no such limit. TS_ERR_HIP if the
 *          array's address cannot be looked up (done once per device, on the
 *          first call with that device current).
 */
ts_status ts_softmax_noalloc(const float* logits, const float* temps, int64_t B, int64_t V,
                             float* out, hipStream_t stream);

/*
 * ts_softmax with an allowed-token mask applied as the logits are read.
 *
 * Defined by: the pull-request page, scope paragraph (allowed-token-ids,
 * min_tokens and grammar masks are what write -inf into the logits) and the
 * test paragraph (the softmax they feed). A disallowed id is treated exactly as
 * a -inf logit, without a separate pass that writes -inf into the logits; the
 * bit layout is this library's.
 *
 * allowed : [B, ceil(V / 32)] uint32, row-major. Id j of row b is allowed when
 *           bit (j % 32) of allowed[b * ceil(V / 32) + j / 32] is 1; bits past
 *           V are ignored. Must not be NULL (use ts_softmax for no mask) and
 *           must not overlap out. Each row needs at least one allowed id with a
 *           finite logit.
 * Others  : as for ts_softmax. The result equals ts_softmax of the logits with
 *           every disallowed id set to -inf, bit for bit.
 */
ts_status ts_softmax_masked(const float* logits, const float* temps, const uint32_t* allowed, int64_t B,
                            int64_t V, float* out, hipStream_t stream);

/*
 * ts_softmax (allowed == NULL) or ts_softmax_masked with the work split
 * forced. Defined by: the pull-request page, bug paragraph (the per-chunk
 * partial and the finalize) and the A/B list (finite rows give the same bits
 * for every kernel configuration with and without the -inf guard, which the
 * tests check over these splits). `variant` is a ts_variant and `chunk` the
 * columns per workgroup (one
 * of 1024, 2048, 4096, 8192, 16384 for SPLIT and FUSED; ignored by ROWWISE;
 * 0 = the table's choice). Same result contract. Meant for tests and tuning; a
 * combination the library cannot run (e.g. FUSED with more chunks per row than
 * it has slots for) returns TS_ERR_INVALID_ARGUMENT.
 */
ts_status ts_softmax_variant(const float* logits, const float* temps, const uint32_t* allowed, int64_t B,
                             int64_t V, float* out, int32_t variant, int32_t chunk, hipStream_t stream);

/*
 * The work split ts_softmax would use for (B, V) on the current device, for a
 * 16-byte aligned call with V % 4 == 0. Host only: launches nothing. Defined
 * by: the pull-request page, A/B script and timing table (the kernel
 * configuration is chosen per shape, there by the autotuner; here by a table
 * measured on MI355X). A row
 * takes the fused split only if the device holds all of its chunks at once;
 * with no HIP device present, that check is skipped (the table alone).
 * variant, chunk : host pointers, written on TS_OK.
 * Errors : TS_ERR_INVALID_ARGUMENT as for ts_softmax, TS_ERR_HIP if the
 *          occupancy query fails.
 */
ts_status ts_plan(int64_t B, int64_t V, int32_t* variant, int32_t* chunk);

/*
 * Inverse-CDF token draws from caller-supplied uniforms.
 *
 * Defined by: the pull-request page, scope paragraph (the sampler consumes the
 * temperature softmax) and results table, sampling row (every draw lands on an
 * allowed id: 1024 of 1024 draws over 16 rows x 64). The page does not give the
 * draw's rule; inverse CDF on caller-supplied uniforms is this library's
 * reading.
 *
 * probs    : [B, V] float32 row-major contiguous, non-negative rows (normally
 *            ts_softmax outputs). Entries that are not > 0 (0, negative, NaN)
 *            are never drawn.
 * uniforms : [B, K] float32. Each u is clamped to [0, 1]; NaN counts as 0.
 * out_ids  : [B, K] int32. For each (b, k): with C the row's inclusive
 *            prefix sums and target = u * C[V-1], the smallest id j with
 *            C[j] > target; for u = 1 the last id with a positive entry.
 *            The row is cut into groups of 4096 ids and each group into
 *            blocks of 64 ids. Prefix sums are integers at three levels: the
 *            groups' float sums at one power-of-two scale per row, the
 *            chosen group's block sums at one scale, then the chosen block's
 *            entries at one scale, each in 64-bit fixed point. Inside a block
 *            the choice is exact; a group or block boundary sits at most
 *            (gamma_12 + gamma_6) / 2 = 5.4e-7 of the row total from the
 *            exact one, gamma_n = n 2^-24 / (1 - n 2^-24) bounding the float
 *            sums over a group (tree depth 12) and a block (depth 6); exact
 *            when every entry is a multiple of one power of two that the sums
 *            hold exactly. The id is always one with a positive entry. A row
 *            with no positive entry (or a sum that is not finite) gives -1.
 * Errors   : TS_ERR_INVALID_ARGUMENT for B < 0, K < 0, V < 1,
 *            V > INT32_MAX, a NULL pointer when B*K > 0, or out_ids overlapping
 *            probs or uniforms. B == 0 or K == 0 is a no-op.
 */
ts_status ts_sample(const float* probs, const float* uniforms, int64_t B, int64_t V, int64_t K,
                    int32_t* out_ids, hipStream_t stream);

/*
 * The softmax and the token draw in one call: ts_softmax followed by
 * ts_sample. Defined by: the pull-request page, scope paragraph (the sampler
 * consumes the softmax) and results table, sampling row (every id drawn has a
 * finite logit). Without probs_out the probabilities are never written: the
 * logits are read once for per-group and per-block partials, and only the
 * 64-id blocks that hold a target are read again.
 *
 * logits, temps : as for ts_softmax.
 * allowed       : NULL, or an allowed-id bitmask as for ts_softmax_masked.
 * uniforms      : [B, K] float32, as for ts_sample.
 * probs_out     : [B, V] float32 or NULL. If not NULL it receives the
 *                 probabilities of ts_softmax (probs_out == logits is
 *                 allowed): the same bits where ts_plan gives the fused or
 *                 split kernels; rows it gives the one-workgroup-per-row
 *                 kernel are computed here by the fused split instead (which
 *                 leaves the draw its group sums), whose bits agree with
 *                 ts_softmax's to the same tolerance. If NULL the
 *                 probabilities are never written.
 * out_ids       : [B, K] int32. The inverse-CDF rule of ts_sample with the
 *                 same three levels of integer prefix sums; every id
 *                 drawn has a finite logit (and an allowed bit); -1 for a row
 *                 with none. With probs_out the draw reads the written
 *                 probabilities (boundaries within 6.9e-7 of the row total of
 *                 those probabilities' exact CDF: the sums are formed before
 *                 scaling, tree depths 14 and 7, and each written value is
 *                 rounded once more); without, it works from the logits (one
 *                 read of them in all), and the float32 exponents add their
 *                 error: at most 3 ln(2) 2^-24 |d| + 5 2^-24 relative per
 *                 entry, |d| its distance below the row's max in log2 units,
 *                 averaged over the row's probabilities.
 * Errors        : as ts_softmax and ts_sample. K == 0 reduces to ts_softmax
 *                 (or a no-op when probs_out is NULL).
 */
ts_status ts_softmax_sample(const float* logits, const float* temps, const uint32_t* allowed,
                            const float* uniforms, int64_t B, int64_t V, int64_t K, float* probs_out,
                            int32_t* out_ids, hipStream_t stream);

/*
 * Not defined by the pages: workspace management. It follows the pattern of
 * the n-gram hash page's "capture-safe" item (fixed shapes, no host reads, no
 * allocation inside a captured replay) so that calls can be captured.
 * Set aside the workspace for any later call with B <= max_B and
 * V <= max_V on `stream`, so that those calls allocate nothing (needed
 * before capturing them into a HIP graph). Allocates and clears device
 * memory; must not itself be called while `stream` is capturing.
 * A graph captured on `stream` keeps using that stream's workspace wherever it
 * is replayed: its replays must not overlap other work on the same workspace
 * (calls on `stream`, or another replay of a graph captured on it), exactly as
 * two calls on one stream never overlap. The workspace lives until the process
 * ends.
 */
ts_status ts_reserve(int64_t max_B, int64_t max_V, hipStream_t stream);

/*
 * Not defined by the pages: diagnostics of this library's fused kernel.
 * Synchronise `stream`, then report and clear the device-side error flags of
 * its workspace. *flags (host pointer) receives the raw bits (bit 0: a fused
 * kernel's bounded wait ran out, and the kernel formed the missing partials
 * itself: the results are exact, the call took the slow path). Returns
 * TS_ERR_SYNC_TIMEOUT if bit 0 was set, else TS_OK.
 */
ts_status ts_device_errors(hipStream_t stream, uint32_t* flags);

/* Not defined by the pages. Static text for a status code (never NULL). */
const char* ts_status_string(ts_status status);

/* Not defined by the pages. TSOFTMAX_ABI_VERSION of the built library. */
int32_t ts_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TSOFTMAX_H_ */
