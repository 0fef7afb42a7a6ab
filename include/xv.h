/*
 * xv.h -- C ABI of libxv, the batch-invariant speculative-decoding verify step
 * for one hybrid (gated-delta-net + attention) layer on AMD Instinct MI355X
 * (gfx950).
 *
 * What the library guarantees.  The r/LocalLLaMA post on bit-exact speculative
 * decoding of Qwen3.8-27B (feedman.me mirror; the paragraph on the two verify
 * changes) makes a k-draft verify reproduce k single-token decode steps bit for
 * bit by running the decode arithmetic in verify: the GDN recurrence through
 * the decode kernel, attention as one decode row per draft position, and (the
 * DeepGEMM paragraph of the same post) small-M projection GEMMs through one
 * tile that gives the same bits at every M.  Every entry point here has ONE
 * code path whose per-row arithmetic does not depend on the number of rows
 * (T or M), the batch size, the row's position in a tile, the cache capacity
 * or the workspace size.  Decode is simply T = 1 (or M = 1).
 *
 * Conventions (all entry points):
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 *  - Every pointer is a DEVICE pointer owned by the caller, dense (C order) in
 *    the stated layout.  Tensors marked [16B] are read or written with 16-byte
 *    vector accesses and must be 16-byte aligned; every other pointer must be
 *    aligned to its element size (2 for bf16, 4 for fp32 / int32), else
 *    XV_ERR_ALIGN.  Nothing is retained after return.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream), allocates nothing and never synchronises.
 *  - Arguments are validated on the host before any launch; a failed check
 *    returns a negative xv_status and launches nothing.  Device-resident values
 *    (kv_len, n_keep) cannot be checked on the host: their preconditions are
 *    stated per call, and kernels clamp them so that no access leaves its
 *    buffer even when a precondition is broken (results are then undefined).
 *  - Stateless and thread-safe; concurrent calls on different streams are
 *    independent as long as their output and workspace buffers do not overlap
 *    (xv_attn_verify_rows_noalloc shares one device array per GPU: see there).
 *    Workspaces carry arrival counters that a call leaves zero for the next.
 *  - An empty problem (B == 0 or M == 0) returns XV_OK and launches nothing.
 */
#ifndef XV_H
#define XV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define XV_ABI_VERSION 8

typedef enum {
    XV_OK = 0,
    XV_ERR_NULL = -1,       /* a required pointer is NULL                         */
    XV_ERR_SHAPE = -2,      /* a size is outside the supported set (see each call) */
    XV_ERR_ALIGN = -3,      /* a pointer breaks its alignment rule                 */
    XV_ERR_WORKSPACE = -4,  /* workspace smaller than xv_attn_workspace_bytes()    */
    XV_ERR_LAUNCH = -5,     /* the HIP runtime rejected a kernel launch            */
    XV_ERR_ALIAS = -6       /* an output buffer is the same as an input it must not overwrite */
} xv_status;

/* Version of this ABI (XV_ABI_VERSION) and a static message for a status code. */
int xv_abi_version(void);
const char* xv_status_string(int status);

/*
 * Small-M projection GEMM:  y[m][n] = bf16( sum_k x[m][k] * w[n][k] ).
 * The post's DeepGEMM paragraph (weights read at a third of DRAM bandwidth at
 * small batch, the fix being a tile that gives the same bits) and the recipe
 * card's runtime env (the M <= 16 gate).
 *
 *   x   : bf16 [M][K]   [16B]  activations (rows = verify rows of all requests)
 *   w   : bf16 [N][K]   [16B]  weights, one output feature per row (K contiguous)
 *   y   : bf16 [M][N]          output, fp32 sum rounded to nearest even
 *   y32 : fp32 [M][N] or NULL  the same sums before rounding
 * Rows are processed in tiles of 16 ([0,16), [16,32), ...; the last may be
 * partial), all tiles against one pass over w.  The bits of row m depend only
 * on x[m][:], w and K: not on M, on the other rows, or on m's place in a tile.
 * Shapes: M >= 0, N >= 16 and N % 16 == 0, K >= 32 and K % 32 == 0.
 */
int xv_gemm_small_m(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                    int M, int N, int K, void* stream);

/*
 * xv_gemm_small_m with its kernel execution timed: start_event and stop_event
 * (hipEvent_t created by the caller, either may be NULL) are recorded when the
 * call's first kernel starts and its last kernel ends, as the launch itself
 * records them (hipExtLaunchKernel), so their interval excludes the dispatch
 * latency that events recorded on the stream around the call include.  Same
 * results, arguments and errors as xv_gemm_small_m; M == 0 launches nothing
 * and records nothing.
 */
int xv_gemm_small_m_timed(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                          int M, int N, int K, void* stream, void* start_event, void* stop_event);

/*
 * Two small-M GEMMs with the same M and K in one launch:
 *   y0 = x0 w0^T ([M][N0]) and y1 = x1 w1^T ([M][N1]),
 * each output bit for bit what xv_gemm_small_m gives it (the same per-block
 * arithmetic; only the launch is shared).  For the decoding step this joins
 * the two projections (x0 = x1) and the two halves of the synthetic head, so
 * the persistent workgroups balance over the union of the column blocks.
 * Where no fused variant exists for the shape (more than 16 rows, or K other
 * than 5120 and 6144) the two GEMMs run one after the other.  start_event /
 * stop_event (hipEvent_t or NULL) are recorded when the first kernel starts
 * and the last one ends, as in xv_gemm_small_m_timed.
 * Arguments, layouts, shapes and errors per GEMM as xv_gemm_small_m; x0 may
 * equal x1.
 */
int xv_gemm_small_m_pair(const uint16_t* x0, const uint16_t* w0, uint16_t* y0, float* y32_0, int N0,
                         const uint16_t* x1, const uint16_t* w1, uint16_t* y1, float* y32_1, int N1,
                         int M, int K, void* stream, void* start_event, void* stop_event);

/*
 * GDN verify: T tokens of the gated delta rule per request, fp32 state.
 * The post, the two verify changes (the GDN recurrence through the decode
 * arithmetic, the old verify kernel having tiled the state differently and
 * kept a different beta precision); the state is fp32 (post, launch command,
 * the mamba SSM dtype flag).  Rule, per value head h (key head g = h / (Hv/Hk)),
 * per token t:
 *     S <- a_t S ;  u = b_t (v_t - S k_t) ;  S <- S + u k_t^T ;  o_t = S q_t
 * which equals S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T.
 * Decode is T = 1; verify of k drafts is T = k + 1.
 *
 *   q, k      : bf16 [B][T][Hk][dk]    [16B] (L2-normalised by the caller)
 *   v         : bf16 [B][T][Hv][dv]
 *   a, b      : fp32 [B][T][Hv]        decay and beta, already activated
 *   state_in  : fp32 [B][Hv][dk][dv]   [16B] S_0, element (value j, key i) at [i][j]; read only
 *   state_out : fp32 [B][Hv][dk][dv]   [16B] S_T; must not be state_in (XV_ERR_ALIAS)
 *   o         : bf16 [B][T][Hv][dv]    outputs o_t rounded to nearest even
 *   o32       : fp32 [B][T][Hv][dv] or NULL
 * Shapes: B >= 0, 1 <= T <= 16, Hk >= 1, Hv % Hk == 0, dk in {64, 128},
 * dv in {32, 64, 96, 128} (multiple of 32, at most 128).
 */
int xv_gdn_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  const float* a, const float* b,
                  const float* state_in, float* state_out,
                  uint16_t* o, float* o32,
                  int B, int T, int Hk, int Hv, int dk, int dv, void* stream);

/*
 * GDN over the T rows of a prompt (prefill; any T >= 1), every row kept: the same
 * per-token arithmetic as xv_gdn_verify, so the outputs and S_T equal T one-token
 * calls bit for bit.  The state stays in registers for the whole call and the rows
 * stream through LDS in blocks of 16.  Arguments, layouts and errors as
 * xv_gdn_verify except 1 <= T < 2^30.
 */
int xv_gdn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const float* a, const float* b,
                   const float* state_in, float* state_out,
                   uint16_t* o, float* o32,
                   int B, int T, int Hk, int Hv, int dk, int dv, void* stream);

/*
 * GDN verify after a verify whose rollback was not run (a lazy rollback: one
 * launch instead of a rollback and a verify).  The previous call ran T_prev
 * rows from state_prev_in to state_prev_out, and n = n_keep_prev[b] of its rows
 * were kept (clamped to [0, T_prev]).  The state of the kept rows is
 *   n == T_prev : state_prev_out (S_T of the previous call; nothing replayed)
 *   otherwise   : S_n, recomputed from state_prev_in over the previous call's
 *                 rows 0..n-1 with the per-token arithmetic of xv_gdn_verify
 * and is written to state_kept; then this call's T rows run from it exactly as
 * in xv_gdn_verify (state_out <- S_T, o and o32 for this call's rows).  Every
 * result equals xv_rollback_to_prefix followed by xv_gdn_verify, bit for bit.
 * The cache length is not touched (xv_greedy_accept's kv_len does that).
 *   q, k, v, a, b, o, o32 : as xv_gdn_verify (this call's rows)
 *   k_prev, v_prev, a_prev, b_prev : the previous call's rows, layouts as k, v, a, b
 *                         with T_prev rows ([16B] k_prev); read only
 *   n_keep_prev         : int32 [B] device
 *   state_prev_in/out   : fp32 [B][Hv][dk][dv] [16B], read only
 *   state_kept          : fp32 [B][Hv][dk][dv] [16B], written
 *   state_out           : fp32 [B][Hv][dk][dv] [16B], written
 * The four states must be distinct buffers (XV_ERR_ALIAS).  Shapes as
 * xv_gdn_verify, and 1 <= T_prev <= 16.  After the last step of a sequence,
 * xv_rollback_to_prefix over the last call's rows leaves the kept state in that
 * call's state_out; it also adds n_keep to its kv_len argument, so pass it a
 * scratch array when xv_greedy_accept has already counted the rows.
 */
int xv_gdn_verify_after(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* a, const float* b,
                        const uint16_t* k_prev, const uint16_t* v_prev,
                        const float* a_prev, const float* b_prev,
                        const int32_t* n_keep_prev, int T_prev,
                        const float* state_prev_in, const float* state_prev_out,
                        float* state_kept, float* state_out,
                        uint16_t* o, float* o32,
                        int B, int T, int Hk, int Hv, int dk, int dv, void* stream);

/*
 * Attention verify rows with the KV append.
 * The post, the two verify changes (verify attention as one decode row per
 * draft position) and the launch command (BF16 KV cache).  Request b holds
 * L0 = kv_len[b] cached positions.  The T new key/value rows are written to
 * cache positions L0..L0+T-1, and row r (query head h, KV head h / (Hq/Hkv))
 * attends positions 0..L0+r:  o = sum_j softmax_j(scale * q.k_j) v_j.
 * The context is split into chunks of xv_attn_chunk_tokens() positions at
 * absolute boundaries; per chunk the partial (max, sum, weighted values) is
 * formed in a fixed order, and the partials are merged in two levels, each in
 * ascending order with a running maximum (a partial that raises it rescales the
 * sums so far): the chunks of each group of 8 consecutive chunks, then the
 * groups.  All of it depends on the row's length and data only, never on T, B,
 * Lmax or the workspace size.
 *
 *   q        : bf16 [B][T][Hq][d]      [16B]
 *   k_new    : bf16 [B][T][Hkv][d]     [16B]  v_new: same
 *   k_cache  : bf16 [B][Hkv][Lmax][d]  [16B]  v_cache: same; rows L0..L0+T-1 are written
 *   kv_len   : int32 [B] device        L0 per request; read only
 *   o        : bf16 [B][T][Hq][d]
 *   o32      : fp32 [B][T][Hq][d] or NULL
 *   workspace: [16B] device scratch of workspace_bytes >= xv_attn_workspace_bytes(B,T,Hq,d,Lmax),
 *              owned by the caller and used by one call at a time.  Its first
 *              4096 bytes are arrival counters: they must be zero before the
 *              first call, and every call leaves them zero (a buffer zeroed once
 *              serves any sequence of calls whose sizes fit).  The rest holds the
 *              chunk partials and needs no initial value.  (When the partials
 *              take the per-tile split, the last of a tile's chunk workgroups to
 *              finish folds that tile's rows in the same launch, a counter
 *              telling it that it is the last; otherwise a second launch folds
 *              every row.)
 *   len_bound: 0, or an upper bound on kv_len[b] + T over the batch, known to
 *              the caller (a serving loop tracks its lengths): the launch is then
 *              sized for that many positions instead of the capacity Lmax (in a
 *              262,144-position cache, rows of a few hundred positions keep the
 *              per-tile split and the shared GDN launch).  The results are the
 *              same bits whatever the bound, as long as it holds; a request with
 *              kv_len[b] + T above a nonzero bound gets undefined outputs (memory
 *              accesses stay within the buffers).
 * Shapes: B >= 0, 1 <= T <= 16, Hq % Hkv == 0, d in {64, 128, 256}, Lmax >= T,
 * ceil(Lmax / chunk) <= 4608, B * Hkv * ceil(Lmax / chunk) * ceil((Hq/Hkv) * T / 16)
 * <= 2^29 (the grid), len_bound == 0 or len_bound >= T
 * (XV_ERR_SHAPE otherwise).  Device precondition: 0 <= L0 and
 * L0 + T <= Lmax (kernels clamp positions to the buffer otherwise).
 * Cache positions >= L0 + T are never read, so they may hold anything.
 */
int    xv_attn_chunk_tokens(void);
size_t xv_attn_workspace_bytes(int B, int T, int Hq, int d, int Lmax);
int    xv_attn_verify_rows(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                           uint16_t* o, float* o32, void* workspace, size_t workspace_bytes,
                           int B, int T, int Hq, int Hkv, int d, int Lmax, float scale,
                           int len_bound, void* stream);

/*
 * xv_attn_verify_rows for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, and the same bits, for calls whose workspace
 * (xv_attn_workspace_bytes(B, T, Hq, d, Lmax)) is at most
 * XV_ATTN_NOALLOC_MAX_BYTES.  The chunk partials go to a device array inside the
 * library (one per GPU it runs on, XV_ATTN_NOALLOC_MAX_BYTES each, held until
 * the process ends); the call allocates nothing.  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (other streams, other host threads)
 * race and give undefined results, so serialise them.  The array is zero when the
 * library is loaded, and every call leaves its arrival counters at zero (the
 * workspace rule of xv_attn_verify_rows); the partials need no initial value.
 * Errors: as xv_attn_verify_rows; XV_ERR_WORKSPACE when the call needs more than
 * XV_ATTN_NOALLOC_MAX_BYTES (checked before any launch); XV_ERR_LAUNCH also when
 * the runtime cannot give the array's address on the current device.
 */
#define XV_ATTN_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int xv_attn_verify_rows_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                uint16_t* o, float* o32,
                                int B, int T, int Hq, int Hkv, int d, int Lmax, float scale,
                                int len_bound, void* stream);

/*
 * GDN verify and attention verify rows in one call.  The two are independent
 * (the post's two verify changes, each with the decode arithmetic) and, at small
 * batch, both are bound by latency rather than bandwidth, so when the attention
 * partials take their per-tile split and both grids fit on the chip at once, one
 * launch runs the GDN workgroups beside the attention partial workgroups (which
 * also fold their rows, as in xv_attn_verify_rows); otherwise the two calls below
 * run one after the other.  Either way every output is bit-identical to
 *   n_keep_prev != NULL : xv_gdn_verify_after(q .. b, k_prev .. b_prev,
 *                         n_keep_prev, T_prev, state_in, state_prev_out,
 *                         state_kept, state_out, o, o32, B, T, Hk, Hv, dk, dv)
 *   n_keep_prev == NULL : xv_gdn_verify(q .. b, state_in, state_out, o, o32,
 *                         B, T, Hk, Hv, dk, dv)  (k_prev .. b_prev, T_prev,
 *                         state_prev_out and state_kept are not used)
 * followed by
 *   xv_attn_verify_rows(q_attn, k_new, v_new, k_cache, v_cache, kv_len, o_attn,
 *                       o_attn32, workspace, workspace_bytes, B, T, Hq, Hkv, d,
 *                       Lmax, scale, len_bound)
 * with each argument's meaning, layout, shape rule and error code as there
 * (the first failing check is reported; nothing is launched then).  The GDN
 * buffers and the attention buffers must not overlap.
 */
int xv_gdn_attn_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const float* a, const float* b,
                       const uint16_t* k_prev, const uint16_t* v_prev,
                       const float* a_prev, const float* b_prev,
                       const int32_t* n_keep_prev, int T_prev,
                       const float* state_in, const float* state_prev_out,
                       float* state_kept, float* state_out,
                       uint16_t* o, float* o32, int Hk, int Hv, int dk, int dv,
                       const uint16_t* q_attn, const uint16_t* k_new, const uint16_t* v_new,
                       uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                       uint16_t* o_attn, float* o_attn32, void* workspace, size_t workspace_bytes,
                       int Hq, int Hkv, int d, int Lmax, float scale,
                       int B, int T, int len_bound, void* stream);

/*
 * Attention of P prompt rows at once (prefill; launch command: chunked prefill).
 * The P new key/value rows are appended at cache positions L0..L0+P-1
 * (L0 = kv_len[b]), then row r attends positions 0..L0+r with
 * exactly the arithmetic of xv_attn_verify_rows for that row (the same chunk
 * partials and the same ordered combine), so every output equals the decode
 * row's bit for bit.  No workspace: each workgroup folds 128 (row, head) pairs'
 * chunk partials in registers, in one pass over the chunks.
 *   q      : bf16 [B][P][Hq][d]  [16B]     k_new, v_new : bf16 [B][P][Hkv][d] [16B]
 *   k_cache, v_cache : bf16 [B][Hkv][Lmax][d] [16B]; rows L0..L0+P-1 are written
 *   kv_len : int32 [B] device; advance != 0: kv_len[b] += P after the rows are formed
 *   o : bf16 [B][P][Hq][d]   o32 : fp32 or NULL
 * Shapes: B >= 0, P >= 1, Hq % Hkv == 0, d in {64, 128, 256}, Lmax >= P,
 * ceil(Lmax / chunk) <= 4608.  Device
 * precondition: 0 <= L0 and L0 + P <= Lmax (positions are clamped otherwise).
 */
int xv_attn_prefill(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                    uint16_t* k_cache, uint16_t* v_cache, int32_t* kv_len,
                    uint16_t* o, float* o32, int B, int P, int Hq, int Hkv, int d, int Lmax,
                    float scale, int advance, void* stream);

/*
 * Rollback to the accepted prefix.
 * The post: the exactness held also with every draft forced to reject and
 * with 8 requests in flight, i.e. keeping any prefix of the verify rows must
 * leave exactly the state sequential decode would have.  For request b with
 * n = n_keep[b] kept rows (0 <= n <= T):
 *   n == T      : state_out already holds S_T; left as is
 *   n == 0      : state_out <- state_in (bit copy)
 *   0 < n < T   : state_out <- S_n, recomputed from state_in over rows 0..n-1
 *                 with the per-token arithmetic of xv_gdn_verify
 *   kv_len[b]  <- kv_len[b] + n
 * The argument arrays are those of the xv_gdn_verify call being rolled back
 * (q is not needed; k, state_in and state_out are [16B]).
 *   state_out : in S_T, out S_n; must not be state_in
 *   kv_len    : int32 [B] device, updated in place
 *   n_keep    : int32 [B] device; values outside [0, T] are clamped
 * Shapes as xv_gdn_verify.
 */
int xv_rollback_to_prefix(const uint16_t* k, const uint16_t* v,
                          const float* a, const float* b,
                          const float* state_in, float* state_out,
                          int32_t* kv_len, const int32_t* n_keep,
                          int B, int T, int Hk, int Hv, int dk, int dv, void* stream);

/*
 * Greedy acceptance at temperature 0 on device (the post compares token ids of
 * greedy decoding, and their logprobs).  logits[b][t][n] = logits_a[...] +
 * logits_b[...] (one fp32 add; logits_b may be NULL).  ids[b][t] = the lowest n
 * among the maxima of row (b, t).  Row t consumed input token draft[b][t]
 * (draft[b][0] is the root); draft t+1 is accepted when it equals ids[b][t] and
 * all earlier drafts were accepted.  n_keep[b] = 1 + accepted drafts (the verify
 * rows to keep, ready for xv_rollback_to_prefix or xv_gdn_verify_after).
 * kv_len (may be NULL): int32 [B] device, kv_len[b] += n_keep[b], the cache
 * length after the kept rows (then no rollback call may add it again).
 * logprob (may be NULL):
 * logprob[b][t] = log softmax(logits[b][t])[ids[b][t]] = -ln sum_n e^(z_n - max z),
 * fp32, in an order fixed by N alone (not by B, T or the pointers' alignment).
 *   logits_a, logits_b : fp32 [B][T][N]     draft : int32 [B][T]
 *   ids : int32 [B][T]   n_keep : int32 [B]   logprob : fp32 [B][T] or NULL
 * Shapes: B >= 0, 1 <= T <= 16, N >= 1.  Logits must be finite.
 */
int xv_greedy_accept(const float* logits_a, const float* logits_b, const int32_t* draft,
                     int B, int T, int N, int32_t* ids, int32_t* n_keep, float* logprob,
                     int32_t* kv_len, void* stream);

/*
 * The synthetic head and greedy acceptance in one call (the post's first
 * paragraph: ids and logprobs of greedy decoding; its DeepGEMM paragraph: the
 * head GEMM bound by reading the weights).  Exactly
 *   xv_gemm_small_m_pair(x_a, w_a, y_a, logits_a, N, x_b, w_b, y_b, logits_b, N, B*T, K)
 *   xv_greedy_accept(logits_a, logits_b, draft, B, T, N, ids, n_keep, logprob, kv_len)
 * bit for bit, every output included.  With B*T <= 16 and K = 5120 or 6144 it is
 * one launch: each workgroup computes one 16-column block of both halves and the
 * block's part of the greedy reduction, and the last workgroup to finish folds
 * them in xv_greedy_accept's order and counts the accepted drafts; otherwise it
 * runs the pair call, then the greedy reduction with the acceptance in the same
 * launch (B <= 63: the last row of each request to finish counts its accepted
 * drafts) or as xv_greedy_accept (more requests).
 *   x_a, x_b : bf16 [B*T][K] [16B]     w_a, w_b : bf16 [N][K] [16B]
 *   y_a, y_b : bf16 [B*T][N]           logits_a, logits_b : fp32 [B*T][N]
 *   draft, ids, n_keep, logprob, kv_len : as xv_greedy_accept
 *   workspace : [16B] device memory of workspace_bytes >=
 *               xv_head_greedy_workspace_bytes(B, T, N), all zero before its
 *               first use; each call returns it with its first 256 bytes zero
 *               again (an arrival counter), so it needs no clearing between
 *               calls.  Calls that share a workspace must not overlap in time
 *               (other streams, other host threads).
 * Inputs and outputs must not overlap.  Shapes: 0 <= B <= 2^20, 1 <= T <= 16,
 * N >= 16 and N % 16 == 0, K >= 32 and K % 32 == 0 (XV_ERR_SHAPE otherwise);
 * XV_ERR_WORKSPACE for a short workspace.  Logits must be finite.
 */
size_t xv_head_greedy_workspace_bytes(int B, int T, int N);
int xv_head_greedy_accept(const uint16_t* x_a, const uint16_t* w_a, uint16_t* y_a, float* logits_a,
                          const uint16_t* x_b, const uint16_t* w_b, uint16_t* y_b, float* logits_b,
                          const int32_t* draft, int32_t* ids, int32_t* n_keep, float* logprob,
                          int32_t* kv_len, void* workspace, size_t workspace_bytes,
                          int B, int T, int N, int K, void* stream);

/*
 * Token embedding rows in front of the projection GEMMs of a decoding step
 * (the post's claim is about whole decoding steps: ids and logprobs of greedy
 * decoding with and without speculation).  x[m][:] = table[tokens[m]][:], a bit
 * copy; ids outside [0, V) are clamped (a precondition the host cannot check).
 *   table  : bf16 [V][H]  [16B]      tokens : int32 [M] device
 *   x      : bf16 [M][H]  [16B]
 * Shapes: M >= 0, V >= 1, H >= 8 and H % 8 == 0.
 */
int xv_embed_rows(const uint16_t* table, const int32_t* tokens, int M, int V, int H,
                  uint16_t* x, void* stream);

/*
 * The per-head operands of the verify calls from the projection rows of one
 * layer (the synthetic layer's column layout; the pages name the model, not
 * its tensors).  Row m of each output depends on row m of y1 and y2 only.
 *   y1 : bf16 [M][N1] [16B]  columns GDN q (Hk*dk) | GDN k (Hk*dk) | GDN v (Hv*dv) | unused
 *   y2 : bf16 [M][N2] [16B]  columns attention q (Hq*d) | k (Hkv*d) | v (Hkv*d) |
 *                            decay logit (Hv) | beta logit (Hv) | unused
 *   q, k   : bf16 [M][Hk][dk] [16B]  u / sqrt(sum u^2 + 1e-6) per head (fp32, fixed order),
 *                                    rounded to nearest even
 *   v      : bf16 [M][Hv][dv] [16B]  a copy
 *   a, b   : fp32 [M][Hv]            a = 1 / (1 + e^alpha) (= exp(-softplus(alpha))),
 *                                    b = 1 / (1 + e^-beta)
 *   q_attn : bf16 [M][Hq][d] [16B], k_new, v_new : bf16 [M][Hkv][d] [16B]  copies
 * With M = B*T these are the [B][T][...] inputs of xv_gdn_verify and
 * xv_attn_verify_rows.  Shapes: M >= 0, dk in {64, 128}, dv and d multiples of
 * 8, N1 and N2 multiples of 8, N1 >= 2*Hk*dk + Hv*dv, N2 >= Hq*d + 2*Hkv*d + 2*Hv.
 */
int xv_split_projections(const uint16_t* y1, const uint16_t* y2, int M, int N1, int N2,
                         int Hk, int Hv, int dk, int dv, int Hq, int Hkv, int d,
                         uint16_t* q, uint16_t* k, uint16_t* v, float* a, float* b,
                         uint16_t* q_attn, uint16_t* k_new, uint16_t* v_new, void* stream);

/*
 * Measurement helper (not part of the verify step): reads bytes0 bytes of src0
 * and bytes1 bytes of src1 once with 16-byte loads, each of sink_words workgroups
 * streaming one contiguous share of their concatenation; workgroup i writes the
 * XOR of the words it read to sink[i] (uint32 [sink_words], device).  start_event / stop_event
 * (hipEvent_t or NULL) are recorded at the kernel's own start and end.  It gives
 * the streaming-read rate of the same bytes a weight-streaming GEMM reads, as the
 * practical ceiling beside the HBM peak.  bytes0, bytes1 multiples of 16,
 * src0, src1 [16B]; XV_ERR_SHAPE / XV_ERR_NULL / XV_ERR_ALIGN otherwise.
 */
int xv_stream_read(const void* src0, size_t bytes0, const void* src1, size_t bytes1,
                   uint32_t* sink, int sink_words, void* stream, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif
#endif /* XV_H */
