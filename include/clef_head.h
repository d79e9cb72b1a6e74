/*
 * libclefhead: JointSchemaHead forward pass on AMD Instinct MI355X (gfx950).
 *
 * The head turns a decision model's final-norm hidden states into one logit
 * per option of every schema question, plus a softmax over each question's
 * options, in one pass with no decoding loop.  Operation as the pages define
 * it:
 *   - "Cloudflare 发布 9B 多模态决策模型 Clef-Flash 完整解析" §三: pool the question
 *     and option spans of the hidden states, route evidence with 2
 *     cross-attention layers, score every option jointly; §四: logits, then a
 *     softmax per question.
 *   - "clef-4bit ... JointSchemaHead" §三 steps 1-4: question vector = mean of
 *     the instruction span; option context = mean of the option span; option
 *     lexical vector = mean of lm_head rows over the option's ids; option
 *     query = sum of three projections; 2 routing layers (cross-attention over
 *     the whole hidden memory + FFN, residual); field vector = question base +
 *     option-weighted summary + global (last) vector + type embedding; 4
 *     transformer layers across fields; logit = prior + gate * (joint_scale *
 *     cosine + residual MLP over [f, o, f*o, |f-o|]).
 *   - CoreML conversion metadata of clef-flash, "decision.head": a LayerNorm
 *     over the hidden width feeds the memory, the global vector is the row at
 *     the final position, spans pool normalised rows; "decision.spans": half-open [start, end) spans that
 *     index the hidden rows; "question_types": noul 0, choice 1, score 2;
 *     "option_order": noul options are [true, false]; "softmax": per question,
 *     fp32, temperature 1.
 *   - Head configuration (architecture page §3.2 table): width 1024, 16 heads,
 *     routing_layers 2, layers 4, feedforward 4096; hidden_size 4096 (5120 for
 *     the 27B variant, clef-4bit page §三).
 *
 * Conventions.
 *   - Every entry point returns 0 (CLEF_OK) on success or a negative CLEF_E_*
 *     code; clef_head_last_error() then holds a message (thread-local).
 *   - All inputs are validated on the host BEFORE anything is launched; on an
 *     error no output buffer is written.
 *   - "HOST" pointers are ordinary CPU memory, read during the call and not
 *     retained.  "DEVICE" pointers are HIP device memory on the current device.
 *   - bf16 means IEEE bfloat16 bit patterns (uint16_t storage).
 *   - No entry point is re-entrant for one handle; distinct handles may be
 *     used from distinct threads.
 */
#ifndef CLEF_HEAD_H
#define CLEF_HEAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CLEF_API __attribute__((visibility("default")))

/* Status codes.  Input errors are raised before any work starts, as the
 * pages' own entry points do: the tuning guide's pitfalls section (an encoded
 * schema longer than the length budget is refused before the state is read)
 * and the clef-4bit page §六 FAQ (a record over the context limit is refused,
 * ContextTooLong / HTTP 413, unless truncation is allowed). */
#define CLEF_OK             0
#define CLEF_E_ARG         -1  /* null pointer, bad config, missing / mis-sized weight (architecture page
                                  §3.2 config table; clef-4bit page §三 names of the head's parts) */
#define CLEF_E_LENGTH      -2  /* record length < 1 or > padded length; mask not a prefix mask (tuning guide
                                  tip 1: collate pads every record on the right to the longest one) */
#define CLEF_E_SPAN        -3  /* empty span, span outside [0, n_b) (CoreML metadata page, decision.spans:
                                  half-open spans over the record's own positions) */
#define CLEF_E_ID          -4  /* token id outside [0, vocab_size) (CoreML metadata page, decision.head
                                  lexical: rows of the untied lm_head table are indexed by the span's ids) */
#define CLEF_E_SCHEMA      -5  /* bad question type, question without options, noul without 2 options
                                  (CoreML metadata page, question_types and option_order) */
#define CLEF_E_NOMEM       -6  /* device or pinned allocation failed */
#define CLEF_E_HIP         -7  /* HIP runtime error (message in clef_head_last_error) */
#define CLEF_E_UNSUPPORTED -8  /* configuration outside what the kernels are built for */

/* weight element types */
#define CLEF_BF16 1
#define CLEF_F32  2

/* batch layouts */
#define CLEF_PADDED 0           /* hidden is [B, L, H]; key_mask gives the valid prefix of each row */
#define CLEF_VARLEN 1           /* hidden is [T, H], records back to back; cu_seqlens gives them */
/* OR'ed into the layout: hidden holds IEEE fp16 elements instead of bf16 (the
 * CoreML packaging hands the head fp16 hidden states and runs the head in
 * fp32: CoreML conversion metadata page of clef-flash, "decision.head",
 * dtype of record).  Row statistics, span pooling and the memory GEMM read
 * fp16 (the GEMM with an fp16 copy of the folded memory weight, fp16 MFMA,
 * fp32 accumulation); everything after the memory rows is unchanged. */
#define CLEF_HIDDEN_F16 0x100

typedef struct clef_head clef_head;   /* opaque handle */

/* Head hyper-parameters (the keys of joint_head_config.json the pages list).
 * The kernels are built for width 1024, 16 heads, feedforward 4096,
 * num_types 3, hidden_size a multiple of 512 up to 8192; routing_layers and
 * layers may be any count >= 0.  ln_eps is the epsilon of every LayerNorm.
 * field_cross_attention selects the reading of the field layers: 0 = pre-LN
 * self-attention across the record's fields + FFN; 1 = the decoder-layer
 * reading (clef-4bit page §三 step 3 and the architecture page §3.2 call them
 * transformer decoder layers): a pre-LN cross-attention of the fields over
 * the record's memory rows between the self-attention and the FFN, with the
 * extra weights P.xln.{w,b}[D], P.{xq,xk,xv,xo}.w[D,D], .b[D] per field layer
 * P, listed after all others. */
typedef struct {
  int32_t hidden_size, width, heads, routing_layers, layers, feedforward, vocab_size, num_types;
  float ln_eps;
  int32_t field_cross_attention;
  int32_t precision;   /* CLEF_PRECISION_BF16 or CLEF_PRECISION_F32, below */
} clef_head_config;

/* Arithmetic of the head, chosen at create (clef_head_config.precision).
 * CLEF_PRECISION_BF16: bf16 storage of the memory rows, K/V rows, routing
 *   queries and attention probabilities, fp32 accumulation, fp32 residual
 *   streams and statistics; activations enter the small products as two bf16
 *   terms (about 16 significant bits).  The head's stored precision (clef-4bit
 *   page §三: its weights are bf16 and never quantised).
 * CLEF_PRECISION_F32: fp32 arithmetic throughout, as the CoreML packaging
 *   runs the head on fp16 hidden states (CoreML conversion metadata page,
 *   decision.head, dtype_of_record): memory rows and K/V in fp32, fp32
 *   attention, and every fp32 value entering a product as three bf16 terms
 *   whose sum is exact, so that each product is exact and only the fp32
 *   accumulation rounds.  The input LayerNorm is applied to fp16 hidden rows
 *   before their product; over bf16 hidden rows (exact as they are) it is
 *   folded into the product's epilogue against the fp32 weight W diag(gamma)
 *   held as three bf16 terms, whose cancellation of the row mean adds about
 *   u |mean| / std relative error (u = 2^-24).  Works with bf16 or fp16
 *   (CLEF_HIDDEN_F16) hidden rows; streamed ingest (clef_head_stream_*) is
 *   CLEF_E_UNSUPPORTED in this mode. */
#define CLEF_PRECISION_BF16 0
#define CLEF_PRECISION_F32  1

/* One named head tensor in host memory.  Linear weights use the [out, in]
 * layout.  Names (D = width, H = hidden_size, F = feedforward):
 *   ln_in.{w,b}[H]; {mem,q_base,q_opt,opt_ctx,opt_lex,glob}.w[D,H], .b[D];
 *   type_emb[num_types,D]; summary.w[D]; summary.b[1];
 *   for P in route.0..route.{routing_layers-1}, field.0..field.{layers-1}:
 *     P.ln1.{w,b}[D]; P.{q,k,v,o}.w[D,D], .b[D]; P.ln2.{w,b}[D];
 *     P.ffn1.w[F,D], .b[F]; P.ffn2.w[D,F], .b[D];
 *   score.w1[D,4D]; score.b1[D]; score.w2[D]; score.b2[1];
 *   gate_logit[1] (CLEF_F32); joint_scale[1] (CLEF_F32).
 * All others are CLEF_BF16.  clef_head_weight_count() and clef_head_weight_info()
 * enumerate them. */
typedef struct {
  const char *name;
  const void *host_data;
  int64_t numel;
  int32_t dtype;
} clef_head_weight;

/* One batch of encoded records.  Spans are record-relative, half-open
 * [start, end), and index the same positions as the hidden rows. */
typedef struct {
  int32_t layout;              /* CLEF_PADDED | CLEF_VARLEN, optionally | CLEF_HIDDEN_F16 */
  int32_t num_records;         /* B >= 1 */
  int32_t max_len;             /* L (CLEF_PADDED): row stride of hidden in rows */
  const void *hidden;          /* DEVICE bf16 (fp16 with CLEF_HIDDEN_F16) [B, L, H] (PADDED) or [T, H] (VARLEN);
                                  padding rows are never read */
  const uint8_t *key_mask;     /* HOST [B, L], 1 = valid; each row must be a prefix mask (PADDED) */
  const int32_t *cu_seqlens;   /* HOST [B+1], cu_seqlens[0] = 0, increasing (VARLEN) */
  int32_t num_questions;       /* NQ >= 0 */
  int32_t num_options;         /* NO */
  const int32_t *q_offsets;    /* HOST [B+1]  records -> questions (CSR) */
  const int32_t *q_type;       /* HOST [NQ]   0 noul, 1 choice, 2 score */
  const int32_t *q_span;       /* HOST [NQ,2] instruction span [start, end) */
  const int32_t *o_offsets;    /* HOST [NQ+1] questions -> options (CSR); option order as in the schema */
  const int32_t *o_span;       /* HOST [NO,2] option description span [start, end) */
  const int32_t *o_ids;        /* HOST [sum of option span lengths] token ids of every option span, in order */
} clef_head_batch;

/* Create a head on the current HIP device (architecture page §3.2: the head's
 * configuration table; clef-4bit page §三: the head's parts, stored in bf16 and
 * never quantised; CoreML metadata page, decision.head: the lexical table is
 * the backbone's untied lm_head, not part of the head).  cfg and weights are
 * HOST memory, read during the call; weights are validated by name, element
 * count and dtype (CLEF_E_ARG on any mismatch, CLEF_E_UNSUPPORTED for a
 * configuration the kernels are not built for), then copied into
 * handle-owned device memory (repacked).  lexical_table is the DEVICE bf16
 * [vocab_size, hidden_size] untied lm_head.weight; it is borrowed and must
 * outlive the handle.  On success *out receives the handle; on any error
 * *out is NULL and nothing is leaked (CLEF_E_NOMEM, CLEF_E_HIP). */
CLEF_API int clef_head_create(const clef_head_config *cfg, const clef_head_weight *weights, int32_t num_weights,
                     const void *lexical_table, clef_head **out);

/* A second head over the same weights (the JointSchemaHead of "clef-4bit ...
 * JointSchemaHead" §三, same operation as clef_head_forward): it reads src's
 * device weight blob and lexical table and has its own workspace and events,
 * so a serving loop can keep several batches in flight, one per head, each on
 * its own stream.  The heads also share the one internal stream on which a
 * forward runs its work that does not wait for the big GEMMs, so n heads in
 * flight need n + 1 streams (HIP gives a process 4 hardware queues by
 * default), and they take turns for the big GEMMs: a forward's memory GEMM
 * starts after the K/V GEMM of the group's previously issued forward, so one
 * batch's GEMMs run beside the other batches' small-GEMM chains.  Results do
 * not depend on this order.  The weight blob and that stream are released with the last head
 * that uses them; src may be destroyed first.  The new head lives on src's
 * device (the current device is left as it was).  Errors: CLEF_E_ARG for NULL
 * src / out, CLEF_E_HIP when events cannot be created (nothing is leaked). */
CLEF_API int clef_head_create_sharing(const clef_head *src, clef_head **out);

/* Forward pass on hip_stream (a hipStream_t, or NULL for the default stream):
 * the whole head of the clef-4bit page §三 steps 1-4 (pool, route, aggregate
 * fields, score), then the per-question softmax of the Clef-Flash overview §四
 * and of the CoreML metadata page's softmax entry (fp32, temperature 1).
 * Outputs (DEVICE, caller-owned): logits fp32 [NO], probs fp32 [NO] (softmax
 * over each question's options), argmax int32 [NQ] (index of the first
 * maximal logit within its question).  The host tables are copied before
 * the call returns; outputs are ready when the stream reaches them.  The
 * handle's workspace grows to the largest batch seen. */
CLEF_API int clef_head_forward(clef_head *h, const clef_head_batch *batch, float *logits, float *probs,
                      int32_t *argmax, void *hip_stream);

/* Answer outputs of clef_head_forward_answers (CoreML conversion metadata page
 * of clef-flash, "decision.response" and "decision.option_order").  Every
 * member is a caller-owned DEVICE fp32 buffer or NULL (then not written):
 *   value          [NQ]  noul: probability of "true" (option 0, the order
 *                        [true, false]); choice: probability of the argmax
 *                        option (the answer itself is argmax[q]); score: the
 *                        probability-weighted mean level, levels 0..n-1
 *   confidence     [NQ]  largest probability of the question (for noul the
 *                        response omits it)
 *   value_4dp, confidence_4dp [NQ], probs_4dp [NO]
 *                        the same numbers and every probability rounded half
 *                        to even at the 4th decimal (the response rounds to four
 *                        decimal places): the fp32
 *                        nearest to k / 10^4, k = the integer nearest to
 *                        x * 10^4 with ties to even, x the fp32 unrounded value.
 * usage.input_tokens of a record is its valid length n_b and output_tokens is
 * 0 (no decoding): both are known to the caller and not written here. */
typedef struct {
  float *value;
  float *confidence;
  float *value_4dp;
  float *confidence_4dp;
  float *probs_4dp;
} clef_head_answers;

/* clef_head_forward plus the answer mapping above, computed in the scoring
 * kernel from the same fp32 probabilities (logits, probs and argmax are
 * bit-identical to clef_head_forward's).  answers must not be NULL
 * (CLEF_E_ARG); otherwise arguments, errors and ownership are those of
 * clef_head_forward. */
CLEF_API int clef_head_forward_answers(clef_head *h, const clef_head_batch *batch, float *logits, float *probs,
                                       int32_t *argmax, const clef_head_answers *answers, void *hip_stream);

/* For callers that cannot allocate device memory (code that sets up HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of clef_head_forward with no device or pinned allocation.  Its workspace is
 * a static array of CLEF_NOALLOC_SCRATCH_BYTES bytes in the library's device
 * code object, which each GPU the library runs on holds from the first such
 * call until the process ends; the host tables are copied from ordinary
 * host memory (the handle keeps a host copy; host-side planning uses the
 * ordinary heap).  Arguments, outputs and errors are those of
 * clef_head_forward, plus CLEF_E_UNSUPPORTED (nothing launched, outputs
 * untouched) when the batch needs more workspace than the array holds (about
 * 16K valid rows at hidden_size 4096: one record at the default max_length
 * 16384 fits), and CLEF_E_ARG while tracing or stage timing is on.  No
 * kernel relies on the array's previous contents, which persist from the
 * last call.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (different streams, or different handles without an
 * order between their streams) race; calls in order on one stream do not. */
#define CLEF_NOALLOC_SCRATCH_BYTES (256ull << 20)
CLEF_API int clef_head_forward_noalloc(clef_head *h, const clef_head_batch *batch, float *logits, float *probs,
                                       int32_t *argmax, void *hip_stream);

/* Streamed ingest: the head consumes a batch's hidden rows while the
 * backbone still produces them (CoreML conversion metadata page of
 * clef-flash, "decision.readout" and "prefill_chunk": a record runs through
 * the backbone as consecutive calls of 64 positions, each returning those
 * positions' final-norm hidden rows), so the head's per-row work (LayerNorm
 * statistics, memory rows, K/V rows of every routing layer) overlaps the
 * backbone and only the option / field / scoring chain remains at the end.
 * The result is bit-identical to clef_head_forward on the same rows.
 *
 * clef_head_stream_begin: batch must use CLEF_VARLEN (cu_seqlens gives each
 *   record's length; CLEF_HIDDEN_F16 may be OR'ed in); batch->hidden is
 *   ignored.  Validates the batch like clef_head_forward (same error codes),
 *   sizes the workspace and handle-owned staging rows [T, H], and uploads the
 *   span tables on hip_stream.  CLEF_E_ARG if a stream is already open.
 * clef_head_stream_rows: rows [row0, row0 + nrows) of record `record`
 *   (DEVICE, nrows x H elements of the batch's element type, row stride H).
 *   Each record's rows arrive in order: row0 must equal the number of its
 *   rows received so far (CLEF_E_ARG otherwise), and rows past its length
 *   are CLEF_E_LENGTH.  The rows are copied on hip_stream (they must stay
 *   valid until the stream reaches the copy); every 256-row tile the chunk
 *   completes is processed at once on hip_stream.
 * clef_head_stream_end: batch must describe the same batch as at begin (its
 *   host tables are read again; CLEF_E_ARG if they differ); every row must
 *   have arrived (CLEF_E_LENGTH otherwise).  Runs the rest of the forward on
 *   hip_stream; outputs as clef_head_forward, plus the answer mapping of
 *   clef_head_forward_answers when answers is not NULL.  The stream is closed
 *   on success.
 * clef_head_stream_cancel: closes an open stream without computing outputs.
 * While a stream is open the handle refuses clef_head_forward (CLEF_E_ARG).
 * Use one HIP stream for a streamed batch, or order the streams. */
CLEF_API int clef_head_stream_begin(clef_head *h, const clef_head_batch *batch, void *hip_stream);
CLEF_API int clef_head_stream_rows(clef_head *h, int32_t record, int32_t row0, int32_t nrows, const void *rows,
                                   void *hip_stream);
CLEF_API int clef_head_stream_end(clef_head *h, const clef_head_batch *batch, float *logits, float *probs,
                                  int32_t *argmax, const clef_head_answers *answers, void *hip_stream);
CLEF_API int clef_head_stream_cancel(clef_head *h);

/* Release everything the handle owns (resource management; no page operation).
 * Waits for the handle's own pending work first.  NULL is ignored. */
CLEF_API void clef_head_destroy(clef_head *h);

/* Message of the last failing call on this thread ("" if none): the text of
 * the raise-early errors above.  The pointer stays valid until the thread's
 * next failing call. */
CLEF_API const char *clef_head_last_error(void);

/* Host-only validation of a batch against a configuration: the same checks
 * clef_head_forward runs before launching.  Writes the total number of
 * valid rows T to *num_rows when num_rows is not NULL.  Needs no GPU. */
CLEF_API int clef_head_check_batch(const clef_head_config *cfg, const clef_head_batch *batch, int64_t *num_rows);

/* Host-only: the pooled row ranges the library derives from a batch.  Writes
 * int32 [NQ + NO + B][2] half-open ranges in packed row space (record b's
 * rows start at the sum of the earlier records' lengths): the instruction
 * span of every question, the description span of every option, then the
 * global row [n_b - 1, n_b) of every record.  Needs no GPU. */
CLEF_API int clef_head_span_rows(const clef_head_config *cfg, const clef_head_batch *batch, int32_t *rows);

/* Host-only: number of named tensors the configuration expects, and the
 * name, element count and dtype of the i-th one. */
CLEF_API int32_t clef_head_weight_count(const clef_head_config *cfg);
CLEF_API int clef_head_weight_info(const clef_head_config *cfg, int32_t i, char *name, int32_t name_cap,
                          int64_t *numel, int32_t *dtype);

/* Debug snapshots of intermediate results of the following forwards.
 * enable != 0 keeps copies; clef_head_trace() copies one to host memory
 * after synchronizing the last forward's stream.  Layouts:
 *   CLEF_TRACE_POOLED  fp32 [NQ + NO + B, H]: question means, option-context means, global rows
 *   CLEF_TRACE_LEXICAL fp32 [NO, H]           option lexical vectors
 *   CLEF_TRACE_PRIOR   fp32 [NO]              lexical prior
 *   CLEF_TRACE_MEMORY  bf16 (fp32 in CLEF_PRECISION_F32) [sum_b ceil(n_b/256)*256, D]:
 *                      record b's rows start at the sum of the earlier records' rounded lengths
 *   CLEF_TRACE_U + r   fp32 [NO, D]           option vectors after r routing layers (r = 0: queries)
 *   CLEF_TRACE_F0      fp32 [NQ, D]           field vectors before the field layers
 *   CLEF_TRACE_F       fp32 [NQ, D]           field vectors after the field layers
 *   CLEF_TRACE_JCOS    fp32 [NO]              joint cosine
 *   CLEF_TRACE_MLP     fp32 [NO]              residual MLP output
 *   CLEF_TRACE_POOL_TABLE int32 [NQ + NO + B'][4], B' = records with questions:
 *                      the pooling entries the kernels read (CoreML metadata page,
 *                      decision.spans): (first row of the span in the hidden buffer's
 *                      own layout, span length, first row in the packed row space,
 *                      output slot) for every question span, then every option span,
 *                      then the global row [n_b - 1, n_b) of every record with questions
 *   CLEF_TRACE_LEX_TABLE int32 [NO][4]: (first position in the id table, id count,
 *                      question slot, global slot) of every option
 *   CLEF_TRACE_IDS     int32 [sum of option span lengths]: the uploaded id table
 * The last three are read back from the device copy the kernels used.
 * bytes must equal the snapshot's size. */
#define CLEF_TRACE_POOLED  1
#define CLEF_TRACE_LEXICAL 2
#define CLEF_TRACE_PRIOR   3
#define CLEF_TRACE_MEMORY  4
#define CLEF_TRACE_F0      5
#define CLEF_TRACE_F       6
#define CLEF_TRACE_JCOS    7
#define CLEF_TRACE_MLP     8
#define CLEF_TRACE_POOL_TABLE 9
#define CLEF_TRACE_LEX_TABLE 10
#define CLEF_TRACE_IDS     11
#define CLEF_TRACE_U       16
CLEF_API int clef_head_set_trace(clef_head *h, int32_t enable);
CLEF_API int clef_head_trace(clef_head *h, int32_t which, void *host_dst, int64_t bytes);

/* Per-stage GPU time of the following forwards, from HIP events recorded on
 * the forward's stream between stages.  enable != 0 turns it on and clears
 * the sums; while on, each forward waits for its own last event before
 * returning.  clef_head_stage_times() writes the summed milliseconds of every
 * stage (ms[CLEF_NUM_STAGES]) and the number of forwards summed. */
#define CLEF_STAGE_ROWSTATS    0   /* LayerNorm statistics of the hidden rows */
#define CLEF_STAGE_POOL        1   /* span means and global rows */
#define CLEF_STAGE_LEXICAL     2   /* lexical gather-mean and prior */
#define CLEF_STAGE_MEMORY_GEMM 3   /* memory projection (hidden width -> 1024) */
#define CLEF_STAGE_KV_GEMM     4   /* K/V projections of every routing layer */
#define CLEF_STAGE_QUERY_PROJ  5   /* option queries, question base, global projections */
#define CLEF_STAGE_ROUTE_DENSE 6   /* routing layers: norms, Q / O / FFN maps */
#define CLEF_STAGE_ROUTE_ATTN  7   /* routing cross-attention and its combine */
#define CLEF_STAGE_FIELD       8   /* field aggregation and field transformer */
#define CLEF_STAGE_SCORE       9   /* residual-MLP hidden layer, scoring, softmax, argmax */
#define CLEF_NUM_STAGES       10
CLEF_API int clef_head_set_profiling(clef_head *h, int32_t enable);
CLEF_API int clef_head_stage_times(clef_head *h, double *ms, int64_t *forwards);

/* Test hooks, process-wide, for exercising failure paths and reads of
 * unwritten memory (no page operation):
 *   CLEF_DEBUG_ALLOC_LIMIT  value = bytes (0: none): every single device or
 *                           pinned allocation the library would make above it
 *                           fails, and the call returns CLEF_E_NOMEM
 *   CLEF_DEBUG_POISON       value != 0: working memory allocated from then on
 *                           (workspace, trace copies, streamed staging rows,
 *                           and the allocation-free scratch at every call) is
 *                           first filled with 0xFFFFFFFF (a NaN in fp32 and
 *                           bf16) by a kernel on the call's stream
 * Returns CLEF_E_ARG for an unknown setting or a negative limit. */
#define CLEF_DEBUG_ALLOC_LIMIT 1
#define CLEF_DEBUG_POISON      2
CLEF_API int clef_head_debug_set(int32_t what, int64_t value);

#ifdef __cplusplus
}
#endif
#endif /* CLEF_HEAD_H */
