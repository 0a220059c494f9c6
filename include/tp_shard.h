/*
 * tp_shard.h -- one tensor-parallel rank's linear share of a Megatron-style
 * transformer layer on an MI355X (gfx950) GPU.
 *
 * The method, after these pages (title, section):
 *   - "Tensor vs Pipeline Parallelism" (xingyuzhitong.com), "Tensor
 *     parallelism: split inside each layer": in the MLP the leading weight
 *     matrix is cut along its output columns and the trailing one along its
 *     input rows; the attention heads are shared out over the ranks; one
 *     all-reduce then adds up the ranks' partial products.
 *   - "AI Infrastructure series, Part 5" (drpranayjha.com), "How does tensor
 *     parallelism split a layer?": attention and MLP are cut the same way
 *     (columns, then rows), so a rank stores and streams 1/N of each matrix;
 *     a 64-query-head model takes 2, 4 or 8 ranks, never 3 or 6, and a group
 *     larger than the 8 key-value heads holds copies of key-value heads.
 *   - "Tensor Parallelism" glossary (aidolsgroup.com), "Full definition":
 *     every rank sees the same input and the ranks' partial products are
 *     added.
 *   - "How do tensor parallelism (TP) and pipeline parallelism (PP) split large
 *     model weights ...?" (iloveeagents.com), "Detail" and "Example": a
 *     4096 x 4096 W cut column-wise into two 4096 x 2048 pieces; a
 *     column-parallel linear keeps out_features / t outputs and computes the
 *     local product.
 *
 * On one GPU the t ranks run one after another, each with its own packed
 * shard and its own fp32 partial, and tp_reduce_partials sums the partials in
 * place of the cross-GPU all-reduce.
 *
 * Conventions for every entry point:
 *   - A weight W is logical [K x N] row-major bf16 (raw uint16_t bits), and a
 *     layer computes Y = X W. "Column" means an output feature.
 *   - bf16 is bfloat16 as raw uint16_t bits. Rounding to bf16 is round to
 *     nearest, ties to even.
 *   - Pointers named "device" point to GPU memory the caller allocated; the
 *     library never allocates, frees or keeps device memory and holds no
 *     state between calls. The caller keeps every buffer alive until the work
 *     queued on `stream` has finished.
 *   - All device work is queued asynchronously on `stream` (a hipStream_t;
 *     NULL means the default stream). No call waits for the GPU.
 *   - Arguments are checked on the host before anything is queued; on any
 *     error nothing is queued and an error code is returned. No C++ exception
 *     crosses this interface. Every call is reentrant.
 *   - Device pointers must be 16-byte aligned; leading dimensions of bf16
 *     arrays must be multiples of 8 elements and those of fp32 arrays
 *     multiples of 4 (TP_ERR_ALIGN otherwise). Inputs and outputs must not
 *     overlap unless a call says otherwise.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define TP_API __attribute__((visibility("default")))
#else
#define TP_API
#endif

typedef struct ihipStream_t* hipStream_t;

typedef int32_t tp_status;
enum {
  TP_OK = 0,
  TP_ERR_NULL = -1,        /* a required pointer is NULL */
  TP_ERR_SHAPE = -2,       /* a size <= 0 (M < 0), or descriptors that do not fit together */
  TP_ERR_INDIVISIBLE = -3, /* t does not divide the split dimension or the heads */
  TP_ERR_RANK = -4,        /* rank outside [0, t) */
  TP_ERR_ALIGN = -5,       /* misaligned pointer, leading dimension or width */
  TP_ERR_WORKSPACE = -6,   /* workspace smaller than tp_workspace_bytes() */
  TP_ERR_HIP = -7,         /* the HIP runtime reported an error at launch */
  TP_ERR_KIND = -8         /* unknown kind, or a kind the call does not take */
};

/* How a rank's shard is cut from the full weight. */
typedef enum {
  TP_COL = 0,        /* columns [r N/t, (r+1) N/t) of W [K x N] */
  TP_ROW = 1,        /* rows    [r K/t, (r+1) K/t) of W [K x N] */
  TP_GATEUP_COL = 2, /* W = [Wg | Wu], N = 2 I: columns [r I/t, (r+1) I/t) of Wg and of Wu */
  TP_QKV_COL = 3,    /* W = [Wq | Wk | Wv], N = (n_q + 2 n_kv) d: the rank's Q, K and V heads */
  TP_O_ROW = 4,      /* W [n_q d x N]: the rows of the rank's Q heads */
  TP_DGRAD = 5       /* the transpose of a planned shard, for its input gradient (tp_shard_plan_dgrad) */
} tp_kind;

/* Which kernel family runs a linear. AUTO picks DECODE for M <= 64. */
typedef enum {
  TP_PATH_AUTO = 0,
  TP_PATH_DECODE = 1,  /* split-K MFMA GEMV, HBM-bound; needs M <= 64 */
  TP_PATH_PREFILL = 2  /* LDS-tiled MFMA GEMM, compute-bound */
} tp_path;

/* How the packed shard stores its weights. */
typedef enum {
  TP_W_BF16 = 0,     /* bf16 values as given */
  TP_W_FP8_E4M3 = 1  /* one byte per weight: OCP FP8 E4M3 codes, one power-of-two scale per output column */
} tp_wformat;

/* Attention shape: query heads, key-value heads, head dimension. */
typedef struct {
  int32_t n_q, n_kv, head_dim;
} tp_heads;

/* A run of columns of the full W: columns [src_col, src_col + len) become
 * shard columns [dst_col, dst_col + len). */
typedef struct {
  int64_t src_col, len, dst_col;
} tp_col_range;

/* One rank's shard (plain old data, filled by tp_shard_plan). */
typedef struct {
  int32_t kind, t, rank, n_col_ranges;
  int64_t K, N;                 /* full logical weight [K x N] */
  int64_t shard_k, shard_n;     /* logical shard [shard_k x shard_n] */
  int64_t row_begin, row_end;   /* rows of W in the shard: [row_begin, row_end) */
  tp_col_range col_ranges[3];   /* columns of W in the shard, in shard order */
  int32_t q_head_begin, q_head_end;   /* attention kinds: the rank's Q heads */
  int32_t kv_head_begin, kv_head_end; /* attention kinds: the rank's KV heads */
  int32_t kv_replicated;        /* 1 if t > n_kv: the KV head is repeated on t / n_kv ranks */
  int32_t path;                 /* tp_path; tp_shard_plan sets TP_PATH_AUTO, the caller may change it */
  int64_t out_n;                /* width of the column output: shard_n, or shard_n / 2 (= I/t) for TP_GATEUP_COL */
  int64_t packed_k, packed_n;   /* padded sizes of the packed layout */
  int64_t packed_bytes;         /* bytes tp_shard_pack writes */
  int32_t wformat;              /* tp_wformat; tp_shard_plan sets TP_W_BF16 (see tp_shard_set_wformat) */
  int32_t reserved;             /* 0 */
} tp_shard_desc;

/*
 * Plans rank `rank` of `t` for a weight of kind `kind`, logical [K x N]
 * (host only, integer, no GPU work). `heads` is required for TP_QKV_COL and
 * TP_O_ROW and ignored otherwise.
 *
 * Rules ("Tensor vs Pipeline Parallelism", "Tensor parallelism: split inside
 * each layer" and "Common mistakes"; "AI Infrastructure series, Part 5",
 * "How does tensor parallelism split a layer?"): t must divide the split
 * dimension exactly, never a ragged split (TP_ERR_INDIVISIBLE). For the
 * attention kinds n_q % t == 0, and n_kv % t == 0 when t <= n_kv, else
 * t % n_kv == 0 and rank r holds KV head floor(r n_kv / t), repeated.
 * TP_QKV_COL needs N == (n_q + 2 n_kv) d, TP_O_ROW needs K == n_q d, and
 * n_q % n_kv == 0 (TP_ERR_SHAPE). The kernels read 16-byte vectors, so the
 * shard's k extent, its output width and d must be multiples of 8
 * (TP_ERR_ALIGN).
 */
TP_API tp_status tp_shard_plan(tp_kind kind, int64_t K, int64_t N, int32_t t, int32_t rank,
                        const tp_heads* heads, tp_shard_desc* out);

/*
 * Switches a planned shard to another weight storage before it is packed
 * ("AI Infrastructure series, Part 5", "Reason 2": a decoded token streams
 * all the weights, 70.6 GB for a 70B model stored in 8 bits, half of its
 * 16-bit size). Sets desc->wformat and recomputes packed_k and
 * packed_bytes; everything else is unchanged.
 *   TP_W_BF16: packed_k = shard_k rounded up to 32, 2 bytes per weight.
 *   TP_W_FP8_E4M3: weight-only 8-bit storage; the activations stay bf16.
 *     Output column n of the shard gets the exponent e_n, the smallest
 *     integer with max_k |W[k][n]| <= 448 * 2^e_n (0 for an all-zero column),
 *     and each weight the OCP FP8 E4M3 code (1 sign, 4 exponent bits with
 *     bias 7, 3 mantissa bits, subnormals, largest finite 448) nearest to
 *     W[k][n] * 2^-e_n, ties to even, sign kept. The linears multiply by the
 *     dequantised weights decode(code) * 2^e_n, which are exact in bf16.
 *     packed_k = shard_k rounded up to 64; packed_bytes = packed_k * packed_n
 *     (codes) + 4 * packed_n (the scales 2^e_n as fp32).
 * Unknown format -> TP_ERR_KIND; an invalid descriptor -> its check's error.
 */
TP_API tp_status tp_shard_set_wformat(tp_shard_desc* desc, int32_t wformat);

/*
 * Copies the rank's shard out of the full weight into the kernels' packed
 * layout ("AI Infrastructure series, Part 5", "What does it look like in vLLM
 * ...": the shards are cut once, while the model is loaded). Load-time work.
 *   W        device, full logical [K x N] bf16, row-major, leading dim ldw >= N
 *   W_packed device, desc->packed_bytes bytes, 16-byte aligned; its layout is
 *            private to the library (tiles of 16 output columns x 32 k for
 *            bf16, x 64 k for 8-bit codes, zero-padded to packed_n x
 *            packed_k, pairs of tiles interleaved by k-step, gate/up tiles
 *            paired; 8-bit shards end with their column scales).
 * For TP_W_FP8_E4M3 the pack quantises as tp_shard_set_wformat states.
 */
TP_API tp_status tp_shard_pack(const tp_shard_desc* desc, const uint16_t* W, int64_t ldw,
                        void* W_packed, hipStream_t stream);

/*
 * Column-parallel linear of one rank ("How do tensor parallelism ... split
 * ...", "Example": each GPU computes its share of the output features as the
 * local product x W_r; "Tensor vs Pipeline Parallelism", "Tensor
 * parallelism: split inside each layer").
 *   X [M x K] bf16, leading dim ldx (every rank reads the same X)
 *   TP_COL, TP_QKV_COL: Y [M x shard_n] = bf16(X W_r) (for QKV the columns
 *     are [Q_r | K_r | V_r])
 *   TP_GATEUP_COL: Y [M x I/t] = bf16(SiLU(X Wg_r) * (X Wu_r)), SiLU(g) =
 *     g / (1 + e^-g): SwiGLU fused into the epilogue, G and U never leave the
 *     GPU's registers
 * Accumulation is fp32 from bf16 products; the result is rounded once to bf16.
 * ldy lets Y be a column slice of a wider buffer. M == 0 queues nothing and
 * returns TP_OK without looking at X, W_packed or Y (they may be NULL).
 * ws: device scratch of at least tp_workspace_bytes(desc, M) bytes, 16-byte
 * aligned, owned by the caller (may be NULL when that is 0); its contents on
 * entry do not matter and on return are undefined. Calls queued on different
 * streams must not share one ws.
 * 8-bit shards (tp_shard_set_wformat): the product uses the dequantised
 * weights decode(code) * 2^e_n with the activations in bf16. The decode path
 * reads the codes and decodes them in registers; the prefill path first
 * writes a bf16 copy of the dequantised shard into ws.
 */
TP_API tp_status tp_col_linear(const tp_shard_desc* desc, const uint16_t* X, int64_t M, int64_t ldx,
                        const void* W_packed, uint16_t* Y, int64_t ldy, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * Row-parallel linear of one rank: the fp32 partial P_r = Z_r W[rows_r, :]
 * ("Tensor vs Pipeline Parallelism", "Tensor parallelism: split inside each
 * layer": second matrix by rows; "Tensor Parallelism" glossary: partial
 * outputs are summed). It never reduces.
 *   Z [M x shard_k] bf16, leading dim ldz: the rank's own input slice (its
 *     column output, or its heads' attention output for TP_O_ROW)
 *   P [M x N] fp32, leading dim ldp
 * Workspace and 8-bit shards as for tp_col_linear.
 */
TP_API tp_status tp_row_linear(const tp_shard_desc* desc, const uint16_t* Z, int64_t M, int64_t ldz,
                        const void* W_packed, float* P, int64_t ldp, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * One rank's feed-forward share: tp_col_linear(gateup) into H, then
 * tp_row_linear(down) from H into the partial P ("AI Infrastructure series,
 * Part 5", "How does tensor parallelism split a layer?": first matrix by
 * columns, second by rows, so the first output slice is exactly the second's
 * input slice and nothing is exchanged between them).
 *   gateup: a TP_GATEUP_COL plan of [Wg | Wu] [H x 2I]; down: a TP_ROW plan of
 *   Wd [I x H] with the same t and rank, and gateup->out_n == down->shard_k
 *   (TP_ERR_SHAPE otherwise).
 *   H_ws device [M x I/t] bf16 (contiguous), P [M x H] fp32 with leading dim ldp.
 *   ws: at least max(tp_workspace_bytes(gateup, M), tp_workspace_bytes(down, M)).
 */
TP_API tp_status tp_ffn_shard(const tp_shard_desc* gateup, const tp_shard_desc* down,
                       const uint16_t* X, int64_t M, int64_t ldx, const void* Wgu_packed,
                       const void* Wd_packed, uint16_t* H_ws, float* P, int64_t ldp,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * tp_ffn_shard for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc. Same
 * arguments, results and errors as tp_ffn_shard, without ws / ws_bytes: the
 * kernels' scratch (split-K fp32 partials) lives in one static device array
 * of TP_NOALLOC_SCRATCH_BYTES per GPU, which the library's code object
 * holds from its first use on that GPU until the process ends. This call
 * allocates nothing. A call whose scratch (the larger of
 * tp_workspace_bytes(gateup, M) and tp_workspace_bytes(down, M)) exceeds
 * TP_NOALLOC_SCRATCH_BYTES returns TP_ERR_WORKSPACE and queues nothing.
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind: calls that may overlap on one GPU (several streams, several host
 * threads) race and must be serialised by the caller. The stream's device
 * must be the calling thread's current device (TP_ERR_HIP otherwise).
 */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
TP_API tp_status tp_ffn_shard_noalloc(const tp_shard_desc* gateup, const tp_shard_desc* down,
                               const uint16_t* X, int64_t M, int64_t ldx, const void* Wgu_packed,
                               const void* Wd_packed, uint16_t* H_ws, float* P, int64_t ldp,
                               hipStream_t stream);

/*
 * The sum that replaces the all-reduce ("Tensor Parallelism" glossary,
 * "Full definition": the ranks' partial products are added; "Tensor vs Pipeline Parallelism": two
 * all-reduces per layer, after attention and after the feed-forward block):
 *   Y[m][n] = P_0[m][n] + P_1[m][n] + ... + P_{t-1}[m][n], added in fp32 in
 *   rank order, where P_r = P + r * stride_elems is [M x N] with leading dim
 *   ldp. Y [M x N] fp32 with leading dim ldy may be P_0 itself (in place);
 *   it must not overlap P_1 ... P_{t-1}. With t == 1 in place (Y == P,
 *   ldy == ldp) the sum is already there and nothing is queued.
 */
TP_API tp_status tp_reduce_partials(const float* P, int64_t stride_elems, int32_t t, int64_t M,
                             int64_t N, int64_t ldp, float* Y, int64_t ldy, hipStream_t stream);

/*
 * Sequence-parallel form of the partial sum ("AI Infrastructure series,
 * Part 5", "What about MoE models and very long prompts?": sequence
 * parallelism splits the parts of a layer that tensor parallelism leaves
 * whole along the sequence, inside the tensor-parallel group). Rank `rank`
 * keeps only its token rows of the summed partials:
 *   Y[i][n] = P_0[rank Mt + i][n] + ... + P_{t-1}[rank Mt + i][n], Mt = M / t,
 * added in fp32 in rank order, so Y is bit for bit rows [rank Mt, (rank+1) Mt)
 * of tp_reduce_partials' result. P_r = P + r * stride_elems is [M x N] fp32
 * with leading dim ldp; Y [Mt x N] fp32 with leading dim ldy must not overlap
 * any P_r. M not divisible by t -> TP_ERR_INDIVISIBLE; rank outside [0, t)
 * -> TP_ERR_RANK. Pointers, N, ldp, ldy and stride_elems: 16-byte aligned /
 * multiples of 4 (TP_ERR_ALIGN). M == 0 queues nothing.
 */
TP_API tp_status tp_reduce_scatter_partials(const float* P, int64_t stride_elems, int32_t t, int64_t M,
                                     int64_t N, int64_t ldp, int32_t rank, float* Y, int64_t ldy,
                                     hipStream_t stream);

/*
 * The gather that goes with it (same passage): before the next
 * column-parallel product every rank needs the whole sequence again, the t
 * ranks' row blocks stacked in rank order:
 *   X[r Mt + i][n] = X_r[i][n],  X_r = Xs + r * stride_elems ([Mt x N] bf16,
 *   leading dim ldb);  X [t Mt x N] bf16 with leading dim ldx.
 * X must not overlap the blocks. Pointers, N, ldb, ldx and stride_elems:
 * 16-byte aligned / multiples of 8 (TP_ERR_ALIGN). Mt == 0 queues nothing.
 */
TP_API tp_status tp_gather_rows(const uint16_t* Xs, int64_t stride_elems, int32_t t, int64_t Mt,
                         int64_t N, int64_t ldb, uint16_t* X, int64_t ldx, hipStream_t stream);

/*
 * Backward of a rank's linear ("Tensor vs Pipeline Parallelism", "Tensor
 * parallelism: split inside each layer": training adds two all-reduces per
 * layer in the backward pass, one per block; "AI Infrastructure series,
 * Part 5", "Why are 8 GPUs not 8 times faster?": training costs 6 x
 * parameters x tokens, the backward twice the forward).
 *
 * Input gradient: dA_r = dC_r W_r^T. tp_shard_plan_dgrad turns the plan of a
 * rank's linear (any kind but TP_DGRAD) into a TP_DGRAD plan of W_r^T:
 * shard_k = fwd->shard_n (the contraction, in the forward shard's column
 * order, [gate | up] for TP_GATEUP_COL), shard_n = out_n = fwd->shard_k;
 * it keeps fwd's rows and column ranges so that tp_shard_pack cuts the
 * transposed shard out of the same full W. tp_row_linear with that plan and
 * its packed copy then computes dA_r [M x fwd->shard_k] in fp32 from dC_r
 * [M x fwd->shard_n] bf16 (for a column layer a partial, summed over the
 * ranks with tp_reduce_partials: the backward all-reduce). bf16 storage only:
 * tp_shard_set_wformat refuses 8-bit for TP_DGRAD (TP_ERR_KIND).
 */
TP_API tp_status tp_shard_plan_dgrad(const tp_shard_desc* fwd, tp_shard_desc* out);

/*
 * Weight gradient of a rank's linear (same passages):
 *   dW[k][n] = sum_m A[m][k] dC[m][n], fp32 [fwd->shard_k x fwd->shard_n],
 *   leading dim lddw, in the forward shard's row and column order;
 *   A [M x fwd->shard_k] bf16 (leading dim lda): the rank's input (X for the
 *   column kinds, its own Z_r for the row kinds); dC [M x fwd->shard_n] bf16
 *   (leading dim lddc): the gradient of the rank's output ([dG | dU] for
 *   TP_GATEUP_COL, the full output gradient for the row kinds).
 * Accumulation is fp32 over the tokens, one MFMA block of 16 or 32 tokens
 * after another in token order (the block size depends on the shard's size
 * only, so a given shape always sums in the same order); dW is overwritten
 * (M == 0 writes zeros). lda, lddc multiples of 8, lddw of 4,
 * pointers 16-byte aligned (TP_ERR_ALIGN).
 */
TP_API tp_status tp_weight_grad(const tp_shard_desc* fwd, const uint16_t* A, int64_t lda,
                         const uint16_t* dC, int64_t lddc, int64_t M, float* dW, int64_t lddw,
                         hipStream_t stream);

/*
 * Gradient through the fused SwiGLU, H = SiLU(G) * U, SiLU(g) = g s,
 * s = 1 / (1 + e^-g) (same passages; the nonlinearity as tp_col_linear's):
 *   dG = dH * U * s * (1 + G (1 - s)),  dU = dH * G * s,
 * evaluated in fp32 and rounded once to bf16 into dGU = [dG | dU]
 * [M x 2w] (leading dim lddgu). GU [M x 2w] bf16 (leading dim ldgu) holds the
 * pre-activations [G | U] (e.g. from two TP_COL plans over the gate and the
 * up half of [Wg | Wu], written side by side with ldy); dH [M x w] fp32
 * (leading dim lddh) is the gradient of H (tp_row_linear with the down
 * projection's TP_DGRAD plan). w, ldgu, lddgu multiples of 8; lddh of 4.
 */
TP_API tp_status tp_swiglu_backward(const uint16_t* GU, int64_t ldgu, const float* dH, int64_t lddh,
                             int64_t M, int64_t w, uint16_t* dGU, int64_t lddgu,
                             hipStream_t stream);

/*
 * Attention core on the rank's heads, with the rank's share of the KV cache
 * ("Tensor vs Pipeline Parallelism", "Tensor parallelism: split inside each
 * layer": the heads are shared out over the ranks, and a rank keeps the KV
 * cache of its own heads only; "AI Infrastructure series, Part 5", "How does
 * tensor parallelism split a layer?": a rank's KV cache is 1/N of the
 * whole, and ranks beyond the key-value head count hold copies of a
 * key-value head; "How do you choose a layout for serving?": Llama 3.1 70B
 * in 16-bit needs 320 KB of KV cache per token). The pages give
 * no formula; the one computed is, per query head of the rank,
 *   softmax(q k^T / sqrt(d)) v
 * over the positions 0..p of its sequence, p its own position (causal), with
 * the key-value head of its group: query head q (global) reads key-value head
 * floor(q / (n_q / n_kv)), which the rank holds (a repeated head when
 * kv_replicated). No position encoding, no bias, no dropout.
 *
 * All of these take the TP_QKV_COL descriptor of the rank; its head
 * dimension d = shard_n / (n_q_r + 2 n_kv_r) must be 64 or 128 (TP_ERR_SHAPE).
 *
 * A batch is S sequences with q_len new tokens each (M = S q_len rows):
 * rows s q_len .. s q_len + q_len - 1 of QKV (the rank's [Q_r | K_r | V_r],
 * bf16, leading dim ldqkv, e.g. tp_col_linear's output) belong to sequence s.
 * kv_len[s] and slot[s] are device int32 arrays: sequence s uses cache slot
 * slot[s] and holds kv_len[s] positions once its new tokens are in, new
 * token i at position kv_len[s] - q_len + i. Slots must be distinct within a
 * call. A sequence with kv_len[s] < q_len, kv_len[s] > max_kv (L_max for the
 * append) or slot[s] outside [0, n_slots) is skipped by tp_kv_append and
 * gets zero output rows from tp_attention; nothing outside the buffers is
 * touched.
 *
 * The caches (K and V apart, caller-allocated, device, 16-byte aligned) are
 * [n_slots x n_kv_r x L_max x d] bf16, position-major per key-value head;
 * L_max d 2 must stay below 2^31 (TP_ERR_SHAPE).
 */

/* Bytes of one cache array (K or V): n_slots n_kv_r L_max d 2; 0 when the
 * descriptor or sizes are invalid. */
TP_API size_t tp_kv_cache_bytes(const tp_shard_desc* qkv, int64_t n_slots, int64_t L_max);

/* Copies the new tokens' K and V rows (the rank's key-value heads) into
 * their positions of their slots. S == 0 is a no-op. */
TP_API tp_status tp_kv_append(const tp_shard_desc* qkv, const uint16_t* QKV, int64_t ldqkv,
                       int32_t S, int32_t q_len, const int32_t* kv_len, const int32_t* slot,
                       uint16_t* Kc, uint16_t* Vc, int64_t n_slots, int64_t L_max,
                       hipStream_t stream);

/*
 * A [M x n_q_r d] bf16 (leading dim lda, a multiple of 8): the rank's query
 * heads side by side, each row the attention of its token over its
 * sequence's cache (which must already hold the new tokens: tp_kv_append
 * first). max_kv (q_len <= max_kv <= L_max) bounds every kv_len entry.
 * Scores and softmax in fp32; the probabilities enter the product with V as
 * two bf16 terms (hi + lo); output rounded once to bf16.
 * When (n_q_r / n_kv_r) q_len <= 16 (decode) the cache is read in chunks of
 * 512, 1024, 2048 or 4096 positions (the longest that still leave 256 or more
 * workgroups), each once per key-value head; with more than one chunk per
 * sequence the chunks' partials (fp32) go to the workspace:
 * tp_attention_workspace_bytes bytes (TP_ERR_WORKSPACE if short or not
 * 16-byte aligned). Otherwise no workspace is used and ws may be null.
 */
TP_API tp_status tp_attention(const tp_shard_desc* qkv, const uint16_t* QKV, int64_t ldqkv,
                       int32_t S, int32_t q_len, const int32_t* kv_len, const int32_t* slot,
                       int32_t max_kv, const uint16_t* Kc, const uint16_t* Vc, int64_t n_slots,
                       int64_t L_max, uint16_t* A, int64_t lda, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Workspace tp_attention needs for these sizes (0 for the prefill form or
 * invalid arguments). */
TP_API size_t tp_attention_workspace_bytes(const tp_shard_desc* qkv, int32_t S, int32_t q_len,
                                    int32_t max_kv);

/* Bytes of device workspace tp_col_linear / tp_row_linear need for this
 * shard at this M: fp32 partial sums when K is split over workgroups (decode
 * batches of 17..64 tokens with few output tiles; prefill shapes whose output
 * tiles alone cannot fill the GPU, or whose last round of tiles would run at
 * most half full), plus the dequantised copy of an 8-bit shard on the prefill
 * path; 0 when the chosen kernels need none or the descriptor is invalid. The value assumes X at its smallest leading
 * dimension (shard_k); a wider one never needs more. tp_ffn_shard needs the
 * larger of its two descriptors' values. */
TP_API size_t tp_workspace_bytes(const tp_shard_desc* desc, int64_t M);

/* A static, human-readable name for a status code. */
TP_API const char* tp_status_str(tp_status status);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
