/*
 * tp_shard.h - one tensor-parallel rank's share of a Llama-style decoder
 * layer's linear path, computed on one AMD Instinct MI355X (gfx950).
 *
 * Every shard of a t-way split lives in the one GPU's HBM. Column-parallel
 * linears (qkv_proj, gate_up_proj, the vocab-parallel LM head) produce the
 * rank's slice of the output; row-parallel linears (o_proj, down_proj)
 * produce partial sums; tp_reduce_partials is the arithmetic of the
 * all-reduce and tp_concat_logits that of the logits all-gather, both over
 * buffers resident in this GPU's memory.
 *
 * Pages cited (title, section):
 *   [P1] "第 9 章 多进程与张量并行", sections 3.1 (communication) and 3.2 (splitting)
 *   [P2] "Tensor Parallelism 执行路径", weight-split diagram and forward flow
 *   [P3] "张量、流水线与数据并行", sections "线性层怎么切" and
 *        "每 token 的通信量（估算）"
 *
 * Conventions shared by every call
 *   Layout     Row-major, contiguous. Weights are stored [out, in], so a linear
 *              computes Y = X W^T and K (the input dimension) is contiguous.
 *              Full fused QKV rows are [Q (n_h d); K (n_kv d); V (n_kv d)];
 *              full fused gate_up rows are [gate (I); up (I)].
 *   Types      Activations and weights are bfloat16; every sum is accumulated
 *              in fp32; every bf16 result is rounded once, to nearest even.
 *              Partials and logits may be fp32 instead (tp_dtype). Token ids
 *              are int32.
 *   Memory     Device pointers unless stated. The caller allocates and owns
 *              every buffer; inputs are never written. Base pointers must be
 *              16-byte aligned. Outputs must not overlap inputs, except that
 *              tp_reduce_partials accepts out == partials[0] (in place).
 *   Streams    `stream` is a hipStream_t (NULL = the null stream). Every device
 *              call is asynchronous on it and does not synchronise.
 *   Workspace  Scratch beyond a call's inputs and outputs (split-K partial
 *              tiles and their arrival counters, the attention's per-chunk
 *              records, an operand a fused call's two-launch path stages) is a
 *              caller-owned device buffer passed as (workspace,
 *              workspace_bytes); the library allocates nothing and keeps no
 *              state between calls. Layout: the first TP_WS_COUNTER_BYTES hold
 *              uint32 arrival counters, which must be zero before the first
 *              call that uses the buffer (zero-fill it once); every call leaves
 *              them zero again. The rest holds fp32 scratch and needs no
 *              initialisation. tp_workspace_bytes() is the size the kernel
 *              choice is tuned for. A smaller buffer (or NULL with size 0)
 *              makes the linears keep K within one workgroup, which always
 *              fits; calls that cannot run without scratch return
 *              TP_ERR_SHAPE. Calls sharing one workspace must be ordered (one
 *              stream, or synchronised): two in flight at once race.
 *   Errors     Arguments are validated on the host before any HIP call; on
 *              failure a negative tp_status is returned and nothing runs.
 *              M == 0 (or numel == 0) is a valid no-op. A launch failure
 *              reported by the runtime is returned as TP_ERR_HIP. No C++
 *              exception crosses this interface.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = -1,          /* a required pointer is NULL                        */
    TP_ERR_SHAPE = -2,         /* negative or inconsistent sizes                    */
    TP_ERR_DIVISIBILITY = -3,  /* a split rule of [P1 3.2] does not hold            */
    TP_ERR_ALIGNMENT = -4,     /* pointer not 16-byte aligned or a size not % 8     */
    TP_ERR_DTYPE = -5,         /* unknown tp_dtype or weight kind                   */
    TP_ERR_RANGE = -6,         /* t outside [1, 64], rank outside [0, t)            */
    TP_ERR_HIP = -7            /* the HIP runtime reported an error                 */
} tp_status;

typedef enum { TP_BF16 = 0, TP_F32 = 1 } tp_dtype;

typedef enum {
    TP_W_QKV = 0,      /* fused qkv_proj   full [(n_h + 2 n_kv) d, H]  column split by heads */
    TP_W_O = 1,        /* o_proj           full [H, n_h d]             row split             */
    TP_W_GATE_UP = 2,  /* fused gate_up    full [2 I, H]               column split          */
    TP_W_DOWN = 3,     /* down_proj        full [H, I]                 row split             */
    TP_W_EMBED = 4,    /* embedding table  full [V, H]                 vocab split, padded   */
    TP_W_LM_HEAD = 5   /* LM head          full [V, H]                 vocab split, padded   */
} tp_weight_kind;

typedef struct {
    int32_t hidden;        /* H   */
    int32_t num_q_heads;   /* n_h */
    int32_t num_kv_heads;  /* n_kv */
    int32_t head_dim;      /* d   */
    int32_t intermediate;  /* I   */
    int32_t vocab;         /* V (unpadded) */
} tp_model_cfg;

#define TP_MAX_SHARDS 64

/* Bytes of arrival counters at the front of a workspace (65536 uint32). */
#define TP_WS_COUNTER_BYTES 262144

/* ------------------------------------------------------------------------
 * Host-only queries. They make no HIP call and work without a GPU.
 * ------------------------------------------------------------------------ */

/* Static message for a tp_status value. Never NULL. */
const char* tp_status_string(int status);

/* Shape [rows, cols] of the full weight of `kind`. */
int tp_full_shape(const tp_model_cfg* cfg, int kind, int64_t* rows, int64_t* cols);

/* Shape [rows, cols] of one rank's shard of `kind` for a t-way split, after
 * checking the split rules of [P1 3.2]: n_h % t == 0; n_kv % t == 0 when
 * n_kv >= t, t % n_kv == 0 when n_kv < t (KV heads replicated); I % t == 0.
 * QKV: (n_h/t + 2 kv) d x H with kv = max(1, n_kv/t); O: H x n_h d/t;
 * GATE_UP: 2I/t x H; DOWN: H x I/t; EMBED / LM_HEAD: ceil(V/t) x H. */
int tp_shard_shape(const tp_model_cfg* cfg, int t, int kind, int64_t* rows, int64_t* cols);

/* Rows per vocab shard: the vocab padded to a multiple of t and split evenly,
 * [P1 3.2] (Vocab Parallel). Returns ceil(vocab / t), or a negative tp_status. */
int64_t tp_vocab_shard_rows(int64_t vocab, int t);

/* KV heads held by `rank`: `count` consecutive heads starting at `first`.
 * count = n_kv / t when n_kv >= t; otherwise count = 1 and the head is
 * rank / (t / n_kv), shared by t / n_kv consecutive ranks, so each rank's
 * query heads keep the KV head of their GQA group ([P1 3.2]; [P3 线性层怎么切],
 * num_kv_head_replicas). */
int tp_kv_heads_of_rank(const tp_model_cfg* cfg, int t, int rank, int* first, int* count);

/* Workspace size the kernel choice is tuned for: TP_WS_COUNTER_BYTES of
 * counters plus 16 MiB of fp32 scratch (enough for every split-K plan of a
 * decode-sized linear and for the decode attention's records at up to
 * B nkv ceil(L / chunk) (nq / nkv) (d + 2) = 4 Mi floats). */
int64_t tp_workspace_bytes(void);

/* Number of tiled kernel shapes a tp_linear_plan's prefill_tile may name
 * (prefill_tile = v + 1 for v in [0, count)). Host only. */
int tp_prefill_tile_count(void);

/* ------------------------------------------------------------------------
 * Device calls
 * ------------------------------------------------------------------------ */

/* S1. Copy rank `rank`'s shard of a full bf16 weight into `shard_w`
 * (shape from tp_shard_shape). [P1 3.2]; [P3 线性层怎么切].
 *   QKV      rows of the rank's n_h/t Q heads, then its KV heads' K rows, then
 *            the same heads' V rows.
 *   GATE_UP  gate rows [r I/t, (r+1) I/t), then up rows I + the same range.
 *   O, DOWN  input columns [r K/t, (r+1) K/t) of every row, packed contiguous.
 *   EMBED, LM_HEAD  rows [r Vs, (r+1) Vs) with Vs = ceil(V/t); rows past V are
 *            written as zeros.
 * full_w: [full rows, full cols] bf16; shard_w: [shard rows, shard cols] bf16.
 * hidden, head_dim and the shard's column count must be multiples of 8. */
int tp_shard_weights(const tp_model_cfg* cfg, int t, int rank, int kind,
                     const void* full_w, void* shard_w, void* stream);

/* S2, S3. Column-parallel linear: y[M, N] = x[M, K] w_shard[N, K]^T (+ bias[N]),
 * bf16 in, fp32 accumulate, bf16 out. The input is replicated, the output is
 * the rank's slice and is not gathered ([P3 线性层怎么切]: gather_output off;
 * [P1 3.2] Column Parallel). bias_or_null: bf16 [N] or NULL. K % 8 == 0. */
int tp_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, int64_t N,
                     const void* bias_or_null, void* y, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* S4. SwiGLU on a rank's fused gate_up output: out[m, j] =
 * silu(gu[m, j]) * gu[m, i_shard + j], silu(g) = g / (1 + e^-g), computed in
 * fp32 and rounded once. gu: [M, 2 i_shard] bf16; out: [M, i_shard] bf16.
 * [P3 线性层怎么切] (SiLU x up between gate_up and down). i_shard % 8 == 0. */
int tp_swiglu(const void* gu, int64_t M, int64_t i_shard, void* out, void* stream);

/* S5, S7. Row-parallel linear, local part: partial[M, N] =
 * x_shard[M, K_shard] w_shard[N, K_shard]^T, fp32 accumulate, stored as
 * `partial_dtype` (TP_BF16 or TP_F32). The partial still needs the sum over
 * ranks ([P1 3.2] Row Parallel; [P2] output_partial). K_shard % 8 == 0. */
int tp_row_linear_partial(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard,
                          int64_t N, void* partial, int partial_dtype, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* S6, S8, S9b. Sum of t partial buffers: out = sum_{i=0}^{t-1} partials[i],
 * accumulated in fp32 in the fixed order i = 0, 1, ..., t-1 starting from
 * partials[0], and rounded once to `out_dtype` ([P1 3.1] All-Reduce:
 * Y = Y_0 + ... + Y_{p-1}). `partials` is a HOST array of t device pointers,
 * each to `numel` elements of `in_dtype`. out may equal partials[0]. */
int tp_reduce_partials(const void* const* partials, int t, int64_t numel, int in_dtype,
                       void* out, int out_dtype, void* stream);

/* S3 + S4 in one call: act[m, j] = silu(g) * u with g = bf16(x[m, :] . w[j, :])
 * and u = bf16(x[m, :] . w[i_shard + j, :]), silu as in tp_swiglu, computed in
 * fp32 and rounded once ([P1 3.2] SwiGLU MLP; [P3 线性层怎么切]: gate_up
 * column-parallel, then SiLU x up on the rank's slice with no exchange).
 * w_gate_up: the rank's [2 i_shard, K] bf16 shard, rows [gate | up] as
 * tp_shard_weights lays them out; act: [M, i_shard] bf16. Gives the same bits
 * as tp_column_linear (no bias) followed by tp_swiglu, without writing the
 * [M, 2 i_shard] intermediate. K % 8 == 0; any i_shard >= 1. */
int tp_column_linear_swiglu(const void* x, int64_t M, int64_t K, const void* w_gate_up, int64_t i_shard,
                            void* act, void* workspace, int64_t workspace_bytes, void* stream);

/* S5 + S6 / S7 + S8 in one call: the row-parallel linear of rank `rank`
 * followed by the sum over ranks ([P1 3.2] Row Parallel then [P1 3.1]
 * All-Reduce): out = bf16(sum_{i=0}^{t-1} P_i) accumulated in fp32 in the
 * order i = 0..t-1 from P_0, where P_i (i != rank) = partials[i] and P_rank =
 * x_shard w_shard^T stored as `partial_dtype` stores it (rounded to bf16 for
 * TP_BF16, the fp32 sum itself for TP_F32). `partials` is a HOST array of t
 * pointers; entry `rank` is ignored (may be NULL), the others are device
 * [M, N] buffers of `partial_dtype` that must not overlap `out`
 * (TP_ERR_SHAPE). out: [M, N] bf16. Gives the same bits as
 * tp_row_linear_partial (partial_dtype) into partials[rank] followed by
 * tp_reduce_partials (bf16 out). One launch, the sum being the linear's
 * epilogue, when N % 4 == 0 and either M <= 64 with t <= 16, or M > 64 with
 * t <= 2, TP_BF16 partials, K_shard % 64 == 0 and no forced plan (the prefill
 * tile's store reads the peer's partial); otherwise the own partial is
 * staged (in `out` for TP_BF16, in the workspace for TP_F32: M N 4 bytes of
 * scratch, TP_ERR_SHAPE if short) and the reducer sums the t buffers. */
int tp_row_linear_reduce(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                         const void* const* partials, int partial_dtype, int t, int rank, void* out,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* Residual add and RMSNorm, replicated on every rank ([P1 3.2]: the norm is
 * not split; every rank applies the whole norm to the whole hidden row;
 * [P3 流水线并行]: the residual travels beside hidden_states). In place on
 * the residual stream: residual[m, :] = bf16(residual[m, :] + x[m, :]) (x may
 * be NULL: no add, residual unchanged), then
 *   out[m, j] = bf16(h[m, j] * r_m * gamma[j]),  r_m = 1 / sqrt(mean_j h[m, j]^2 + eps)
 * with h the new residual, all in fp32 (the mean is a fixed-order sum, the
 * same run to run). x, residual, out: [M, H] bf16; gamma: [H] bf16; eps finite
 * and >= 0 (TP_ERR_RANGE otherwise); H % 8 == 0, H <= 32768 (TP_ERR_SHAPE:
 * one workgroup holds a row in registers). out, residual, gamma and x
 * must not overlap (TP_ERR_SHAPE). */
int tp_add_rmsnorm(const void* x_or_null, int64_t M, int64_t H, void* residual, const void* gamma, float eps,
                   void* out, void* stream);

/* S6 / S8 + residual add + RMSNorm in one call: the sum over ranks of a
 * row-parallel output ([P1 3.1] All-Reduce, as tp_reduce_partials: fp32 in
 * the order i = 0..t-1 from partials[0], rounded to bf16), added to the
 * residual and normalised as tp_add_rmsnorm does. `partials` is a HOST array
 * of t >= 1 device pointers to [M, H] buffers of `partial_dtype`; none may
 * overlap residual or out. Gives the same bits as tp_reduce_partials (bf16
 * out) followed by tp_add_rmsnorm. */
int tp_reduce_add_rmsnorm(const void* const* partials, int t, int partial_dtype, int64_t M, int64_t H,
                          void* residual, const void* gamma, float eps, void* out, void* stream);

/* The decode layer's norm folded into its neighbours, so that the per-layer
 * step is four launches, not six ([P1 3.2]: the norm is replicated on every
 * rank; [P3 流水线并行]: the residual travels beside hidden_states).
 *
 * tp_row_linear_reduce_add: tp_row_linear_reduce's sum over ranks (the
 * rank's partial x_shard W^T stored as `partial_dtype` stores it, summed in
 * fp32 from rank 0 in order, rounded once to bf16) added to the residual
 * stream in place:
 *   residual[m, n] = bf16(residual[m, n] + that sum)
 * - the same bits as tp_row_linear_reduce into a buffer followed by
 * tp_reduce_add_rmsnorm's residual update. `partials` as in
 * tp_row_linear_reduce (host array of t device pointers of `partial_dtype`,
 * slot `rank` ignored); none may overlap residual ([M, N] bf16). One launch
 * when M <= 64, t <= 16 and N % 4 == 0; otherwise two (the rank's partial is
 * staged in the workspace: M N 2 or 4 bytes of scratch; then N % 8 == 0 and
 * N <= 32768, TP_ERR_SHAPE otherwise).
 *
 * tp_fold_norm_weight (load time, like tp_shard_weights): the norm's gamma
 * folded into the next linear's weight, w_folded[n, k] = bf16(w[n, k] *
 * gamma[k]) ([N, K] bf16, K % 8 == 0; w_folded may equal w, no other
 * overlap), so that RMSNorm(h) W^T = r (h w_folded^T) with a per-row r.
 *
 * tp_rmsnorm_column_linear / tp_rmsnorm_column_linear_swiglu: the column
 * linear (tp_column_linear, tp_column_linear_swiglu) of RMS-normalised rows,
 * given the folded weight:
 *   y[m, n] = r_m sum_k h[m, k] w_folded[n, k],  r_m = 1 / sqrt(mean_k h[m, k]^2 + eps)
 * (= RMSNorm(h) gamma W^T up to the rounding of the folded weight), the
 * normalised rows never written. h: [M, K] bf16 (the residual stream, read
 * only); eps finite and >= 0 (TP_ERR_RANGE); K <= 32768. When M <= 64 and
 * the decode kernel's plan stages X in LDS, the norm is folded into it: the
 * sums of squares come from the diagonal of h h^T on the matrix cores and r
 * scales the outputs (one launch at M <= 16, K split across workgroups as
 * the plain linear would be or whole rows of K <= 5120 in one; at 17-64
 * tokens one launch, or two when K is split: the partial tiles with each
 * split's share of the sums of squares, then the sum that applies r).
 * Otherwise two: tp_add_rmsnorm's kernel (unit weights) writes bf16(h r)
 * into the workspace (M K 2 bytes of scratch must fit, TP_ERR_SHAPE
 * otherwise), then the plain linear reads it. y / act must not
 * overlap h (TP_ERR_SHAPE). */
int tp_fold_norm_weight(const void* w, int64_t N, int64_t K, const void* gamma, void* w_folded, void* stream);
int tp_row_linear_reduce_add(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                             const void* const* partials, int partial_dtype, int t, int rank, void* residual,
                             void* workspace, int64_t workspace_bytes, void* stream);
int tp_rmsnorm_column_linear(const void* h, float eps, int64_t M, int64_t K, const void* w_folded, int64_t N,
                             const void* bias_or_null, void* y, void* workspace, int64_t workspace_bytes,
                             void* stream);
int tp_rmsnorm_column_linear_swiglu(const void* h, float eps, int64_t M, int64_t K, const void* w_gate_up_folded,
                                    int64_t i_shard, void* act, void* workspace, int64_t workspace_bytes,
                                    void* stream);

/* One decode step of the rank's grouped-query attention, with the KV-cache
 * append ([P2 前向执行的实际流程] Step 2: each rank computes attention for its
 * own heads with no exchange; [P2 KV Cache 在 TP 下怎样分布]: each rank holds
 * and writes only its own KV heads; [P3 线性层怎么切]: a KV head shared by
 * several ranks is replicated in each). Sequence b's new token (its K and V
 * in the qkv row) is written to position lens[b] of the cache, then
 *   ctx[b, h d + j] = sum_{p <= lens[b]} softmax_p(q_h . k_p / sqrt(d)) v_p[j]
 * with Q head h reading KV head h / (nq / nkv); fp32 math, one rounding.
 * No rotary embedding is applied. qkv: [B, (nq + 2 nkv) d] bf16, rows
 * [Q heads | K heads | V heads] (tp_column_linear's output with the
 * tp_shard_weights QKV layout); k_cache, v_cache: [B, nkv, L, d] bf16 (read,
 * and written at lens[b]); lens: DEVICE [B] int32, read on the device: a
 * sequence with lens[b] outside [0, L) gets a zero ctx row and no cache
 * write; ctx: [B, nq d] bf16, head h in columns [h d, (h+1) d) — the rank's
 * o_proj input. d in {32, 64, 128, 256}, nq % nkv == 0, nq / nkv <= 8,
 * L <= 32768, B <= 65535 (TP_ERR_SHAPE otherwise). Two launches on the
 * stream: one workgroup per (chunk of 192 cache positions, 64 at d = 256;
 * KV head; sequence) writes a partial record, then the records of each
 * (sequence, head) are combined in chunk order. The records live in the
 * workspace's scratch: B nkv ceil(L / chunk) (nq / nkv) (d + 2) floats must
 * fit (TP_ERR_SHAPE otherwise; the counters are not used). */
int tp_decode_attention(const void* qkv, int64_t B, int nq, int nkv, int head_dim, void* k_cache, void* v_cache,
                        int64_t L, const int32_t* lens, void* ctx, void* workspace, int64_t workspace_bytes,
                        void* stream);

/* S9a. Vocab-parallel embedding, one shard's contribution: for each token m,
 * out[m, :] = e_shard[ids[m] - rank Vs, :] when rank Vs <= ids[m] <
 * min((rank+1) Vs, vocab), else a row of -0.0 (Vs = ceil(vocab / t)). Ids
 * outside [0, vocab) are masked in every shard, so padded rows are never
 * read. Summing the t contributions with tp_reduce_partials reproduces the
 * direct lookup bit for bit, since -0.0 is an exact additive identity
 * ([P1 3.2] Vocab Parallel; [P3 线性层怎么切], embedding then all-reduce).
 * ids: [M] int32; e_shard: [Vs, H] bf16; out_partial: [M, H] bf16; H % 8 == 0. */
int tp_vocab_embed(const int32_t* ids, int64_t M, const void* e_shard, int64_t vocab, int t,
                   int rank, int64_t H, void* out_partial, void* stream);

/* S10. LM-head shard: logits_shard[M, v_shard] = h[M, K] w_lm_shard[v_shard, K]^T,
 * fp32 accumulate, stored as `out_dtype`; padded rows of the shard (zeros)
 * give zero logits. Only sampled positions are passed in ([P3 线性层怎么切]:
 * each card computes V/t logits for the positions to be sampled). */
int tp_lm_head_shard(const void* h, int64_t M, int64_t K, const void* w_lm_shard, int64_t v_shard,
                     void* logits_shard, int out_dtype, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* S11. Concatenate t shard logits in vocab order and drop the padding:
 * out[m, r v_shard + j] = shard_logits[r][m, j] for r v_shard + j < vocab
 * ([P1 3.1] All-Gather, Y = cat(Y_0, ..., Y_{p-1})). `shard_logits` is a HOST
 * array of t device pointers to [M, v_shard] buffers of `dtype`; out is
 * [M, vocab] of the same dtype. v_shard must equal ceil(vocab / t). */
int tp_concat_logits(const void* const* shard_logits, int t, int64_t M, int64_t v_shard,
                     int64_t vocab, int dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Every linear through one call, with an explicit kernel plan
 * ------------------------------------------------------------------------ */

/* Epilogue of a linear (tp_linear_call.epilogue). */
typedef enum {
    TP_EPI_STORE = 0,       /* y = x w^T (+ bias), stored as out_dtype: tp_column_linear,
                               tp_row_linear_partial, tp_lm_head_shard                        */
    TP_EPI_SWIGLU = 1,      /* w holds 2 n rows [gate | up], y = SwiGLU, [M, n] bf16:
                               tp_column_linear_swiglu                                        */
    TP_EPI_REDUCE = 2,      /* y = the sum over ranks: tp_row_linear_reduce                   */
    TP_EPI_REDUCE_ADD = 3   /* y (the residual) += the sum over ranks: tp_row_linear_reduce_add */
} tp_epilogue;

/* Which kernel shape runs a linear. A zero-filled plan is the automatic
 * choice the named calls make. decode_* (M <= 64; all zero = automatic):
 * the decode kernel with `decode_ksteps` 32-wide k steps per wave,
 * `decode_nwn` waves along the output rows (16 rows each), `decode_nwk` waves
 * along K per workgroup, K split across as many workgroups as it takes to
 * cover it, and `decode_x_direct` = 1 to load activation fragments per wave
 * instead of staging them in LDS. prefill_tile (0 = automatic, v + 1 =
 * tiled kernel v, which then runs at any token count M, decode sizes
 * included, except for the reduce epilogues): 0, 1, 2 = 256 x 256,
 * 256 x 128, 128 x 128 tiles (weight rows x tokens) with 32-wide k-tiles on
 * 4 waves; 4, 5, 6 the same on 8 waves; 7 = 192 x 128 on 4 waves;
 * 8, 9, 10 = 256 x 256, 256 x 128, 128 x 128 on 8 waves with 64-wide
 * k-tiles (K % 64 == 0); 11 = 192 x 128 likewise; 12, 13 = 64 x 64 and
 * 128 x 64 on 4 waves and 14 = 64 x 64 on 2 waves, 64-wide k-tiles (tiles
 * for 64 tokens); 15 = 128 x 128 on 4 waves with two 64-wide stages (two
 * workgroups per CU); 16 = 192 x 256 on 8 waves (the last weight rows of a
 * product whose 256 x 256 tiles make between one and two waves); 17 =
 * 128 x 256 on 8 waves with three 64-wide stages; 3 = register-staged
 * 128 x 128 (any K % 8). A decode shape
 * that is not built for any token count, or a prefill_tile outside
 * [0, tp_prefill_tile_count()], is TP_ERR_RANGE. A plan this call cannot run
 * (the shape not built for its token count, an X chunk beyond LDS, split
 * partials beyond the workspace, a K multiple not met) is replaced by the
 * automatic choice; results then differ only in the fp32 summation order.
 * Every tiled shape but 3, and the decode shapes with decode_x_direct = 1,
 * address their operands with 32-bit byte offsets: a weight or activation of
 * 4 GiB or more runs those tiles on shape 3 instead (same bits), and the
 * per-wave decode plan is not used for it. */
typedef struct {
    int32_t decode_ksteps, decode_nwn, decode_nwk, decode_x_direct;
    int32_t prefill_tile;
} tp_linear_plan;

/* Arguments of tp_linear_ex. Every field has the meaning, layout and checks
 * of the named call the epilogue (and `norm`) selects:
 *   x [M, K] bf16; w [N, K] bf16 (TP_EPI_SWIGLU: [2 n, K] with n = N);
 *   bias [N] bf16 or NULL (TP_EPI_STORE only); y [M, N] of out_dtype
 *   (TP_EPI_SWIGLU: [M, n] bf16; TP_EPI_REDUCE_ADD: the residual, in place);
 *   partials / partial_dtype / t / rank: the other ranks' partials (host
 *   array, slot rank ignored) for the two reduce epilogues;
 *   norm = 1 with eps: x's rows RMS-normalised, gamma folded into w
 *   (tp_rmsnorm_column_linear(_swiglu); TP_EPI_STORE and TP_EPI_SWIGLU only);
 *   plan: the kernel shape (tp_linear_plan); workspace as for every call. */
typedef struct {
    const void* x;
    int64_t M, K;
    const void* w;
    int64_t N;
    const void* bias;
    void* y;
    int32_t out_dtype;
    int32_t epilogue;
    const void* const* partials;
    int32_t partial_dtype, t, rank;
    int32_t norm;
    float eps;
    tp_linear_plan plan;
    void* workspace;
    int64_t workspace_bytes;
} tp_linear_call;

/* Run the linear `call` describes on `stream`: what the named call of its
 * epilogue computes, with the kernel shape of call->plan. For sweeps and
 * for tests that run every kernel variant; the named calls are this call
 * with the automatic plan. */
int tp_linear_ex(const tp_linear_call* call, void* stream);

/* ------------------------------------------------------------------------
 * Without allocation or workspace
 * ------------------------------------------------------------------------ */

/* For callers that can neither allocate nor pass device memory of their own
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): tp_column_linear without the workspace argument. Its split-K
 * scratch is a fixed array in the library's device memory, one copy per GPU,
 * held until the process ends: TP_WS_COUNTER_BYTES of arrival counters and
 * 4 MiB of fp32 partials. The call takes the kernel plan tp_column_linear
 * takes with a workspace of tp_workspace_bytes() and gives the same bits;
 * when that plan's partials (splits x M x N floats) exceed 4 MiB it returns
 * TP_ERR_SHAPE and launches nothing. All calls on one GPU share that GPU's
 * array: calls that overlap on one GPU (different streams or host threads)
 * race; calls ordered on one stream do not. The first call on a device also
 * launches a small kernel on `stream` that clears the counters. Arguments and
 * errors otherwise as tp_column_linear. */
int tp_column_linear_noalloc(const void* x, int64_t M, int64_t K, const void* w_shard, int64_t N,
                             const void* bias_or_null, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
