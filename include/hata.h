/*
 * hata.h -- C ABI of libhata.so, the HATA decode-step hot path on MI355X (gfx950).
 *
 * HATA (Hash-Aware Top-k Attention; paper notes "HATA: Trainable and
 * Hardware-Efficient Hash-Aware Top-k Attention for Scalable Large Model
 * Inference", ACL 2025, arXiv 2506.02572).  Each decode step of one attention
 * layer does, per (sequence b, KV head h) "unit":
 *   1. HashEncode the new query rows and the new key row: project by the KV
 *      head's W_H, take the sign, bit-pack into r-bit codes
 *      (section "Key design: Decode-stage algorithm"; hash function from
 *      "Learning-to-Hash modelling");
 *   2. append the key code to the unit's code cache;
 *   3. Hamming distance popcount(q_code XOR k_code) against every cached code,
 *   4. summed over the G = Hq/Hkv query heads sharing the KV head (GQA);
 *   5. keep the top-k tokens (smallest summed distance) and run exact softmax
 *      attention over the gathered K/V rows only (section "Overall framework",
 *      decode phase; section "Hardware-efficient optimisation": fused encode,
 *      XOR+popcount scoring, gather fused into the attention kernel).
 *
 * Conventions fixed here (the notes leave them open):
 *   - bit c of a code is 1 iff the fp32 projection p_c compares >= 0.0f
 *     (so -0.0 gives 1 and NaN gives 0; the matrix-core encode of long row
 *     runs reads the sign of its fp32 accumulator, the same bit for every
 *     finite input since that sum never ends at -0.0, unspecified for NaN
 *     inputs); bit c lives in 32-bit word c/32 at bit position c%32 (for
 *     r >= 64 equally in 64-bit word c/64 at bit c%64);
 *   - one W_H per KV head, stored [Hkv][d][r] row-major, used for the G query
 *     heads of that KV head and for its keys; query head j uses KV head j/G;
 *   - the kept set is the first min(k, n) tokens in (summed distance, token
 *     index) ascending order -- ties go to the lower index -- reported in
 *     ascending token order and padded with -1;
 *   - attention logits are scale * <q, K_i> with softmax over the kept rows
 *     only; outputs are fp32.
 *
 * Layouts (all contiguous, row-major; bf16 arrays are passed as const void*):
 *   q      bf16   [B][Hq][d]
 *   K, V   bf16   [B][Hkv][cap][d]          (row n_b-1 is the new token)
 *   W_H    fp32   [Hkv][d][r]
 *   codes  uint32 [B][Hkv][cap][r/32]       (16-byte aligned; bit c of a code
 *            is bit c % 32 of word c / 32, so for r >= 64 a row is also
 *            r/64 little-endian 64-bit words)
 *   out    fp32   [B][Hq][d]
 *   idx    int32  [B][Hkv][k]
 *   seq_lens int32 [B] on the device: n_b, the number of valid rows
 *            including the new token.  max_len is a host-side upper bound of
 *            every n_b, used only to size launch grids (so calls can be
 *            captured in a HIP graph); it must satisfy 1 <= max_len <= cap.
 *
 * Supported sizes: d = 128; r in {32, 64, 128, 256} (a code of r bits takes
 * r/32 32-bit words, r/8 bytes: 4 at r = 32; hata_sparse_decode and
 * hata_dense_decode take no code); G = Hq/Hkv in {1, 2, 4, 8};
 * 1 <= k <= 4096.
 *
 * Ownership and threading: every pointer is a device pointer unless stated;
 * the caller allocates and owns every buffer, the library never allocates,
 * frees or keeps a pointer after returning, creates no stream and never
 * synchronises (hata_workspace_check, a diagnostic, is the one call that
 * waits for its stream).  `stream` is a hipStream_t passed as void* (NULL =
 * default stream).
 * Workspaces are sized by hata_workspace_bytes, zeroed once by the caller
 * (hata_workspace_reset), restore their own state at the end of every call
 * and must not be shared by calls that can run concurrently.
 *
 * Errors: every call validates its host-side arguments first and returns a
 * hata_status without launching anything if they are bad (outputs are left
 * untouched).  HATA_ERR_HIP reports a failed launch.  Device-side values
 * (seq_lens entries, idx entries) are bounds-checked inside the kernels:
 * out-of-range rows are skipped, never dereferenced.  No C++ exception
 * crosses this interface.  hata_last_error_message() gives a thread-local
 * description of the last failure.
 */
#ifndef HATA_H_
#define HATA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HATA_OK = 0,
  HATA_ERR_NULL = 1,        /* a required pointer is NULL */
  HATA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes */
  HATA_ERR_UNSUPPORTED = 3, /* sizes outside the supported set (d, r, G, k) */
  HATA_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
  HATA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  HATA_ERR_HIP = 6          /* the HIP runtime reported an error */
} hata_status;

/* Operation ids for hata_workspace_bytes. */
enum {
  HATA_OP_TOPK = 1,
  HATA_OP_SPARSE_DECODE = 2,
  HATA_OP_DECODE_STEP = 3,
  HATA_OP_DENSE_DECODE = 4,
  HATA_OP_DECODE_STEP_PAGED = 5
};

/* Static description of a status code. */
const char* hata_status_string(int status);

/* Thread-local detail of the most recent failed call on this thread. */
const char* hata_last_error_message(void);

/* Library version as major*10000 + minor*100 + patch. */
int hata_version(void);

/*
 * HashEncode and append (decode-stage steps 1-2; fused projection, sign,
 * bit-pack and cache update).
 * x is bf16 [B][H][x_rows][d]; for each (b, h) and j in [0, n_new) the row
 * p_b + j of x is encoded with W_H[h / (H/Hkv)] and written to row p_b + j of
 * codes [B][H][cap][r/32], where p_b = pos ? pos[b] : 0 (pos: device int32[B]).
 *   queries:      x = q, H = Hq, x_rows = 1, cap = 1, pos = NULL, n_new = 1
 *   key append:   x = K cache, H = Hkv, x_rows = cap, pos = seq_lens - 1 (device)
 *   prefill bulk: x = K cache, H = Hkv, x_rows = cap, pos = NULL, n_new = n
 *                 (large n_new runs on the matrix cores, bit-identical on
 *                 inputs whose fp32 projections are exact)
 * Rows with p_b + j outside [0, min(x_rows, cap)) are skipped.
 * Requires H % Hkv == 0; codes 16-byte aligned.
 */
int hata_encode_append(const void* x, int64_t x_rows, int B, int H, int n_new,
                       const float* W_H, int Hkv, int d, int r, uint32_t* codes,
                       int64_t cap, const int32_t* pos, void* stream);

/*
 * Hamming scores with GQA sum (decode-stage steps 3-4):
 * scores[b][h][i] = sum over g in [hG, hG+G) of popcount(q_codes[b][g] XOR
 * k_codes[b][h][i]) for i < n_b; entries i >= n_b are not written.
 * q_codes uint32 [B][Hq][r/32]; k_codes uint32 [B][Hkv][cap][r/32];
 * scores uint16 [B][Hkv][cap].  Values lie in [0, G*r].
 */
int hata_hamming_scores(const uint32_t* q_codes, const uint32_t* k_codes, int B,
                        int Hq, int Hkv, int r, int64_t cap,
                        const int32_t* seq_lens, int64_t max_len,
                        uint16_t* scores, void* stream);

/*
 * Top-k selection (decode-stage step 5, selection): idx[b][h][0:min(k,n_b)] =
 * ascending token ids of the first min(k, n_b) tokens in (score, id) order;
 * idx[b][h][min(k,n_b):k] = -1.  scores as produced by hata_hamming_scores,
 * every valid entry <= max_score (max_score = G*r; larger values are clamped
 * to max_score).  ws (optional): with at least hata_workspace_bytes(
 * HATA_OP_TOPK, B, Hq, Hkv, d, r, max_len, k) bytes (any contents, G*r >=
 * max_score), sequences longer than 4096 tokens are selected by many
 * workgroups each (chunk histograms, threshold, chunk counts, ordered
 * compaction); without it (NULL or smaller) one workgroup per unit does it.
 * The result is the same either way.
 */
int hata_topk(const uint16_t* scores, int B, int Hkv, int64_t cap,
              const int32_t* seq_lens, int64_t max_len, int k, int max_score,
              int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * Gather + exact sparse attention (decode-stage step 5, attention; gather
 * fused into the attention kernel): for query head j of unit (b, h = j/G),
 * out[b][j] = softmax(scale * q[b][j] K_I^T) V_I over I = the entries of
 * idx[b][h][0:k] that lie in [0, cap) (negative entries are padding).  A
 * unit with no valid entry gets out = 0.
 * ws: hata_workspace_bytes(HATA_OP_SPARSE_DECODE, ...).
 */
int hata_sparse_decode(const void* q, const void* K, const void* V, int B,
                       int Hq, int Hkv, int d, int64_t cap, const int32_t* idx,
                       int k, float scale, float* out, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * The whole decode step in one launch: encode the new queries, encode and
 * append the new key, Hamming + GQA sum over the unit's cache, top-k, gather
 * and exact sparse attention.
 * On entry K/V rows [0, n_b) are valid (row n_b-1 is the new token, written
 * by the caller) and codes rows [0, n_b-1) are valid; on return codes row
 * n_b-1 holds the new key's code, out holds the attention output and, if
 * idx_out is not NULL, idx_out [B][Hkv][k] holds the kept set exactly as
 * hata_topk reports it.  Results are bit-identical to the staged calls
 * (hata_encode_append, hata_hamming_scores, hata_topk) for codes and idx.
 * A sequence whose length (read on the device) lies outside [1, cap] gets
 * out = 0 and idx_out = -1 and its code rows are left unchanged.
 * ws: hata_workspace_bytes(HATA_OP_DECODE_STEP, ...), zeroed once before
 * first use.  A workspace serves the B and Hkv it was zeroed for, at any
 * Hq, r, max_len and k within its size (calls that run the separate
 * kernels leave the fused step's flags alone); before a call with another
 * B or Hkv it must be zeroed again, since the per-unit exchange slots then
 * sit at other offsets.
 * Shapes whose per-unit scores do not fit on chip run the same
 * steps as separate kernels inside this call (idx_out may still be NULL:
 * the kept list then lives in the workspace).
 * The workgroups of one unit exchange histogram windows and partial
 * attention records through the workspace and wait for each other; they
 * must all be resident at once, which the launch size ensures on an
 * otherwise idle device.  Every such wait is bounded (2^22 polls, or the
 * bound set by hata_workspace_set_spin_limit).  A wait that gives up sets
 * bit 0 of the workspace error word (hata_workspace_check) and the unit's
 * results are marked instead of computed from incomplete data: NaN in
 * out (at least the outputs the timed-out workgroup merges) and -2 in
 * idx_out.  The workspace must then be reset (hata_workspace_reset) before
 * its next use.  Kernels of other streams that occupy compute units while
 * a step runs can delay its workgroups' start; the step then waits for
 * them, and fails as above only if they do not start within the bound.
 */
int hata_decode_step(const void* q, const void* K, const void* V,
                     const float* W_H, uint32_t* codes, int B, int Hq, int Hkv,
                     int d, int r, int64_t cap, const int32_t* seq_lens,
                     int64_t max_len, int k, float scale, float* out,
                     int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * hata_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments, layouts and results, with no
 * workspace argument.  Its workspace is a static device array of the
 * library (16 MiB per device, held until the process ends; its address is
 * looked up once per device with hipGetSymbolAddress); the call allocates
 * nothing.  Each call first clears the array's flag slots with a fill
 * kernel on `stream`, so calls of different sizes may follow each other.
 * Every call on one device shares that device's array: calls that can
 * overlap (other streams, other host threads) race and must be serialised
 * by the caller.  Sizes whose workspace (hata_workspace_bytes(
 * HATA_OP_DECODE_STEP, ...)) exceeds 16 MiB are rejected with
 * HATA_ERR_WORKSPACE before anything is launched.  The bounded waits have
 * the default bound; a wait that gives up marks the outputs as for
 * hata_decode_step (the next call clears the flags again).
 */
int hata_decode_step_noalloc(const void* q, const void* K, const void* V,
                             const float* W_H, uint32_t* codes, int B, int Hq,
                             int Hkv, int d, int r, int64_t cap,
                             const int32_t* seq_lens, int64_t max_len, int k,
                             float scale, float* out, int32_t* idx_out,
                             void* stream);

/*
 * hata_decode_step with independent query and key encoders (HashAttention
 * summary page, "Approach": separate query and key encoders): the G query
 * rows of KV head h are encoded with W_Hq[h] and the appended key row with
 * W_Hk[h] (both [Hkv][d][r] fp32, device); the cache rows [0, n_b-1) must
 * hold W_Hk codes (build them with hata_encode_append and W_Hk).  With
 * W_Hk == W_Hq this is hata_decode_step.  Same layouts, workspace, errors
 * (HATA_ERR_NULL also for a NULL W_Hk) and results contract.  In the fused
 * path only the workgroup that owns the appended row loads W_Hk.
 */
int hata_decode_step_qk(const void* q, const void* K, const void* V,
                        const float* W_Hq, const float* W_Hk, uint32_t* codes,
                        int B, int Hq, int Hkv, int d, int r, int64_t cap,
                        const int32_t* seq_lens, int64_t max_len, int k,
                        float scale, float* out, int32_t* idx_out, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Prefill of a prompt (HATA notes, "Method", "Overall framework", second
 * stage: attention computed as usual while the keys are encoded and the
 * codes cached).  For every sequence b with n_b = min(seq_lens[b], max_len)
 * prompt tokens at positions 0..n_b-1:
 *   out[b][h][i] = sum_{j <= i} softmax_j(scale * q[b][h][i] . K[b][h/G][j])
 *                  * V[b][h/G][j]          (causal, fp32 result)
 *   codes[b][g][j] = HashEncode(K[b][g][j], W_H[g]) for j < n_b
 * (the same codes as hata_encode_append), formed from the key tiles the
 * attention has staged, so the prompt keys are read from HBM once.
 * Layouts (device memory): q bf16 [B][Hq][q_rows][d]; K, V bf16
 * [B][Hkv][cap][d] (rows 0..n_b-1 hold the prompt); W_H fp32 [Hkv][d][r];
 * codes uint32 [B][Hkv][cap][r/32]; seq_lens int32 [B]; out fp32
 * [B][Hq][q_rows][d].  Rows at positions >= n_b of out and codes are left
 * as they are.  The weights of the value product are rounded to bf16 (as
 * flash attention does); the scores, the softmax statistics and all
 * accumulation are fp32.  d = 128; r in {32, 64, 128, 256}; G = Hq / Hkv in
 * {1, 2, 4, 8}; 1 <= max_len <= min(q_rows, cap); q, K, V, out 16-byte
 * aligned, codes 8-byte aligned.  No workspace.  Errors: HATA_ERR_NULL,
 * _SHAPE, _UNSUPPORTED, _ALIGN as for the decode step, HATA_ERR_HIP on a
 * launch failure.
 */
int hata_prefill(const void* q, const void* K, const void* V,
                 const float* W_H, uint32_t* codes, int B, int Hq, int Hkv,
                 int d, int r, int64_t q_rows, int64_t cap,
                 const int32_t* seq_lens, int64_t max_len, float scale,
                 float* out, void* stream);

/*
 * hata_prefill into a paged cache: the prompt's K/V rows are read from, and
 * its code rows written to, pools addressed through a block table, as in
 * hata_decode_step_paged (row j of sequence b lives in page
 * block_table[b * max_pages + j / page_rows]; K_pool, V_pool bf16
 * [num_pages][Hkv][page_rows][d], code_pool uint32
 * [num_pages][Hkv][page_rows][r/32]; page ids clamped into
 * [0, num_pages)).  q and out keep hata_prefill's layouts.  The results are
 * those of hata_prefill on the gathered contiguous cache (bit for bit; the
 * same kernel reads its rows through the table).  page_rows a power of two
 * in [16, 65536]; max_len <= max_pages * page_rows; alignments and errors
 * as for hata_prefill.  No workspace.
 */
int hata_prefill_paged(const void* q, const void* K_pool, const void* V_pool,
                       const float* W_H, uint32_t* code_pool,
                       const int32_t* block_table, int max_pages,
                       int num_pages, int page_rows, int B, int Hq, int Hkv,
                       int d, int r, int64_t q_rows, const int32_t* seq_lens,
                       int64_t max_len, float scale, float* out,
                       void* stream);

/*
 * hata_decode_step over a paged cache (the block-table layout of
 * PagedAttention, which the HATA notes build on; their decode step is
 * unchanged): row j of sequence b lives in page block_table[b * max_pages +
 * j / page_rows] of three pools that share the table,
 *   K_pool, V_pool bf16 [num_pages][Hkv][page_rows][d]
 *   code_pool uint32    [num_pages][Hkv][page_rows][r/32]
 * block_table int32 [B][max_pages] (device); page ids outside
 * [0, num_pages) are clamped into it (reads and writes stay in the pools;
 * the results for such rows are then unspecified).  The logical capacity is
 * cap = max_pages * page_rows; seq_lens[b] in [1, max_len], max_len <= cap.
 * Same steps and results as hata_decode_step on the gathered contiguous
 * cache: the key row n_b-1 is encoded and its code written through the
 * table, every code row 0..n_b-1 is scored, top-k by (score, index), and
 * the attention gathers the kept K/V rows through the table.  When the
 * step fits on chip (any r), it runs as hata_decode_step's single kernel
 * (page ids of each workgroup's rows loaded with its first loads);
 * otherwise as separate kernels (row encode, Hamming scan, top-k, gather
 * attention).  page_rows a power of two in [16, 65536]; q, the pools
 * 16-byte aligned; idx_out [B][Hkv][k] optional.  ws: hata_workspace_bytes(
 * HATA_OP_DECODE_STEP_PAGED, ...), zeroed once before first use (as for
 * hata_decode_step).
 */
int hata_decode_step_paged(const void* q, const void* K_pool,
                           const void* V_pool, const float* W_H,
                           uint32_t* code_pool, const int32_t* block_table,
                           int max_pages, int num_pages, int page_rows, int B,
                           int Hq, int Hkv, int d, int r,
                           const int32_t* seq_lens, int64_t max_len, int k,
                           float scale, float* out, int32_t* idx_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Dense flash-decode baseline over all n_b rows of every unit (the same
 * attention with the kept set = every token), same layouts.
 * ws: hata_workspace_bytes(HATA_OP_DENSE_DECODE, ...).
 */
int hata_dense_decode(const void* q, const void* K, const void* V, int B,
                      int Hq, int Hkv, int d, int64_t cap,
                      const int32_t* seq_lens, int64_t max_len, float scale,
                      float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement utility, not part of the decode path: read `bytes` of device
 * memory at `src` once with streaming 16-byte loads (one workgroup per CU,
 * each over a contiguous segment) and fold them into sink (one word per
 * workgroup, at most 1024 words written; words past the CU count are left
 * as they are, so a caller folding sink clears it first).
 * Timing it gives the HBM read rate a plain kernel reaches on this device,
 * against which the decode step's bytes/s can be compared besides the
 * published peak.  src 16-byte aligned, bytes a multiple of 16; sink is a
 * device buffer of sink_words >= 1024 uint64 (HATA_ERR_WORKSPACE if fewer).
 */
int hata_stream_read(const void* src, size_t bytes, uint64_t* sink,
                     size_t sink_words, void* stream);

/*
 * Training pairs for the hash weights (HATA notes, "Key design",
 * "Learning-to-Hash modelling", training-data construction): for sampled
 * query j (row j of q [J][d] bf16, sitting at position q_pos[j] of the
 * sequence, clamped into [0, n)), its keys 0..q_pos[j] of k [n][d] bf16 are
 * scored by the fp32 dot product q.k and ranked (higher score first, ties to
 * the lower key index); the first P = max(1, ceil((q_pos[j] + 1) *
 * pos_permille / 1000)) are positives, labelled s_max for the first down to
 * s_min for the P-th linearly in rank (s_max alone when P = 1), the others
 * -1.  labels [J][n] fp32 (device): row j holds those labels for keys
 * 0..q_pos[j] and 0 beyond.  The pages use the top 10% (pos_permille = 100)
 * and labels in [1, 20].  d = 128; 1 <= n <= 8192 (HATA_ERR_UNSUPPORTED
 * above); q_pos is a device int32[J].  q and k 16-byte aligned, labels
 * 4-byte aligned (HATA_ERR_ALIGN otherwise).
 */
int hata_hash_labels(const void* q, const void* k, const int32_t* q_pos, int J,
                     int n, int d, int pos_permille, float s_max, float s_min,
                     float* labels, void* stream);

/*
 * One gradient step on one head's hash weights W [d][r] fp32 (device, updated
 * in place), HATA notes, "Key design", "Learning-to-Hash modelling": with the
 * relaxed hash h(x) = 2 Sigmoid(sigma x W) - 1 the loss is
 *   eps * sum_j sum_{i <= q_pos[j]} labels[j][i] * ||h(q_j) - h(k_i)||^2
 * + eta * sum_j ||sum_{i <= q_pos[j]} h(k_i)||^2 + lam * ||W^T W - I_r||_F
 * (the Frobenius norm taken unsquared) and the step is W -= lr * dL/dW, all
 * in fp32.  loss [4] fp32 (device) receives the total and the three terms
 * before the step; grad [d][r] (device, nullable) the gradient.  labels as
 * hata_hash_labels writes them; d = 128; r a multiple of 32 up to 256.
 * ws: hata_hash_train_workspace_bytes(J, n, d, r) bytes (contents not
 * kept between calls).
 */
int hata_hash_train_step(const void* q, const void* k, const int32_t* q_pos,
                         const float* labels, int J, int n, int d, int r,
                         float sigma, float eps, float eta, float lam, float lr,
                         float* W, float* grad, float* loss, void* ws,
                         size_t ws_bytes, void* stream);

/* Workspace bytes of hata_hash_train_step (0 for unsupported sizes). */
size_t hata_hash_train_workspace_bytes(int J, int n, int d, int r);

/* Workspace bytes for operation `op` at these sizes (0 if none is needed). */
size_t hata_workspace_bytes(int op, int B, int Hq, int Hkv, int d, int r,
                            int64_t max_len, int k);

/* Zero a workspace on `stream` (a fill kernel, safe under graph capture). */
int hata_workspace_reset(void* ws, size_t ws_bytes, void* stream);

/*
 * Testing aid for the bounded waits of hata_decode_step,
 * hata_decode_step_qk and hata_decode_step_paged: the waits of calls that
 * use this workspace give up after `polls` polls (0 restores the default of
 * 2^22).  Written by a kernel on `stream`; hata_workspace_reset also
 * restores the default.  ws_bytes >= 8.
 */
int hata_workspace_set_spin_limit(void* ws, size_t ws_bytes, uint32_t polls,
                                  void* stream);

/*
 * Synchronise `stream` and read the workspace's device-side error word:
 * *err_out = 0 if no kernel reported a problem since the last reset, else a
 * bit set (1 = a cross-workgroup wait of a decode step gave up after its
 * spin limit; the affected units' outputs are then NaN and their idx_out
 * entries -2, see hata_decode_step).  Diagnostic only; never needed on the
 * hot path.
 */
int hata_workspace_check(const void* ws, size_t ws_bytes, int* err_out,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HATA_H_ */
