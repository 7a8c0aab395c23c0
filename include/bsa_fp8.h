/*
 * bsa_fp8.h -- C ABI of the block-sparse FP8 (E4M3) attention prefill library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (the attention formula of "Quant Block Sparse Attention",
 * section "Operator introduction"; the block mask and its tiling from the
 * hpc-ops block-sparse FP8 attention article, section "Block-sparse
 * scheduling"):
 *
 *   for every sequence b, query head h and query t of that sequence,
 *     Omega_t = { key j < Lkv_b : block_mask[b, h, t/128, j/128] != 0
 *                                 and (causal ? j <= Lkv_b - Lq_b + t : true) }
 *     score_j = softmax_scale * (q[t,h,:]*qscale[t,h]) . (k_j*kdescale_j)
 *     out[t,h,:] = sum_{j in Omega_t} softmax_j(score) * v_j * vdescale_g
 *     lse[h,t]   = ln sum_{j in Omega_t} exp(score_j)
 *   with g = h / (Hq/Hkv).  An empty Omega_t gives out = 0 and
 *   lse = -FLT_MAX ("Quant Block Sparse Attention", section "Sparse indices &
 *   PA page table").  Causal alignment is bottom-right ("right-context causal",
 *   its constraint table).
 *
 *   The probabilities of each 128-key tile, taken against the running row
 *   maximum, are multiplied by 256 and rounded to E4M3 before the P.V product
 *   (hpc-ops article, section "FP8 Tensor Core compute: fixed P-scale
 *   quantisation"); the 1/256 is folded into the final normalisation together
 *   with the V descale.  Active KV tiles are visited in ascending order; tiles
 *   that the mask switches off are never read (hpc-ops article, section
 *   "Active tile list").
 *
 * Ownership and threading
 *   Every array argument is a DEVICE pointer owned by the caller.  The library
 *   allocates no memory, never synchronises, and never reads device data on the
 *   host: a call validates its static arguments on the host, then enqueues its
 *   kernels on `stream` (a hipStream_t; NULL = the null stream) and returns --
 *   one kernel, except where an entry point below says otherwise.  Results are
 *   ready when that stream reaches the end of the call's last kernel.
 *
 * Errors
 *   A call returns BSA_OK (0) or a positive bsa_status.  Static-argument errors
 *   are detected before any HIP call; then nothing is enqueued and the outputs
 *   are untouched.  BSA_ERR_LAUNCH means the HIP launch itself failed.
 *   Data-dependent preconditions (listed below) are not checked, because the
 *   host never reads device memory.
 */
#ifndef BSA_FP8_H
#define BSA_FP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantisation schemes (hpc-ops article, section "FP8 Tensor Core compute",
 * the two QuantType values; "Quant Block Sparse Attention", "Key parameters"). */
typedef enum {
    /* Q per (token, head); K per tensor; V per tensor.
     * qscale float [T, Hq]; kscale float [1]; vscale float [1]. */
    BSA_QUANT_Q_TOKHEAD_K_TENSOR_V_TENSOR = 0,
    /* Q per (token, head); K per (token slot, kv-head); V per kv-head.
     * qscale float [T, Hq]; kscale float laid out like the cache minus the
     * head dimension: [num_pages, page_size, Hkv] (NHD) or
     * [num_pages, Hkv, page_size] (HND); vscale float [Hkv]. */
    BSA_QUANT_Q_TOKHEAD_K_TOKHEAD_V_HEAD = 1
} bsa_quant_type;

/* Paged KV cache layouts (hpc-ops article, section "3.16x": NHD and HND). */
typedef enum {
    BSA_KV_NHD = 0, /* kcache/vcache E4M3 [num_pages, page_size, Hkv, 128] */
    BSA_KV_HND = 1  /* kcache/vcache E4M3 [num_pages, Hkv, page_size, 128] */
} bsa_kv_layout;

typedef enum {
    BSA_OK = 0,
    BSA_ERR_NULL_POINTER = 1,  /* a required pointer (or dims) is NULL          */
    BSA_ERR_HEAD_DIM = 2,      /* head_dim != 128                               */
    BSA_ERR_PAGE_SIZE = 3,     /* page_size not 32 or 64 (decode: below 1)      */
    BSA_ERR_GQA = 4,           /* Hq % Hkv != 0 or Hq/Hkv outside 1..16         */
    BSA_ERR_QUANT_TYPE = 5,    /* quant_type not a bsa_quant_type               */
    BSA_ERR_KV_LAYOUT = 6,     /* kv_layout not a bsa_kv_layout                 */
    BSA_ERR_SIZE = 7,          /* a size is negative or inconsistent            */
    BSA_ERR_MASK_SHAPE = 8,    /* mask_tiles_q * 128 < max_seqlen_q, or a mask
                                  dimension is not positive                     */
    BSA_ERR_SOFTMAX_SCALE = 9, /* softmax_scale not finite; for the prefill and
                                  the schedule also negative                    */
    BSA_ERR_TOO_LARGE = 10,    /* mask_tiles_kv above BSA_MAX_KV_TILES, or a
                                  grid dimension overflow                       */
    BSA_ERR_LAUNCH = 11,       /* the kernel launch failed                      */
    BSA_ERR_Q_LAYOUT = 12,     /* options->q_layout not a bsa_q_layout          */
    BSA_ERR_P_SCALE = 13,      /* options->p_scale not 0 and not in (0, 448]    */
    BSA_ERR_SPARSE_FORM = 14,  /* block_mask and sparse_indices both given, or
                                  only one of sparse_indices / sparse_seq_len   */
    BSA_ERR_SCHEDULE = 15,     /* schedule_len does not match the task count    */
    BSA_ERR_SCALE_MODE = 16,   /* scale_mode not a bsa_scale_mode               */
    BSA_ERR_QK_PRECISION = 17, /* options->qk_precision not a bsa_qk_precision  */
    BSA_ERR_SCRATCH = 18       /* the partial results do not fit the library's
                                  static scratch (BSA_DECODE_SCRATCH_BYTES)     */
} bsa_status;

/* How bsa_fp8_quantize_append computes a descale from a row's largest
 * magnitude (FlashMLA FP8 KV-cache article, "Quant/dequant source"). */
typedef enum {
    BSA_SCALE_AMAX = 0,      /* d = amax / 448 (float32 division)              */
    BSA_SCALE_AMAX_POW2 = 1  /* d = amax / 448 rounded up to a power of two    */
} bsa_scale_mode;

/* Query layouts ("Quant Block Sparse Attention", "Key parameters": layout_q). */
typedef enum {
    BSA_Q_TND = 0, /* q E4M3 [T, Hq, 128], qscale float [T, Hq] */
    BSA_Q_NTD = 1  /* q E4M3 [Hq, T, 128], qscale float [Hq, T] */
} bsa_q_layout;

/* Matrix path of the Q.K^T products of the prefill.  The hpc-ops article
 * ("FP8 Tensor Core compute") runs both products on FP8 matrix units.  On
 * gfx950 the FP8 products sum 8 consecutive terms at a time with each term
 * aligned to the largest exponent sum of the eight and cut below 2^-13 of
 * it, so they keep fewer bits than an fp32 sum does; the f16 path widens the
 * E4M3 operands exactly and sums with fp32-like accuracy.  The split FP8 path
 * gives each K operand two FP8 products: one with the query codes within two
 * binades of the largest magnitude a lane holds, one with the rest (+0 where
 * the other product has the code), which keeps large and small terms out of
 * the same group of eight.  All feed the same softmax, P quantisation and
 * FP8 P.V product. */
typedef enum {
    BSA_QK_DEFAULT = 0,   /* the library's choice (BSA_QK_FP8_SPLIT)           */
    BSA_QK_F16 = 1,       /* E4M3 widened exactly to f16, f16 matrix products */
    BSA_QK_FP8 = 2,       /* E4M3 operands, one FP8 product per K operand     */
    BSA_QK_FP8_SPLIT = 3  /* E4M3 operands, two FP8 products per K operand    */
} bsa_qk_precision;

/* Largest block-mask width (KV tiles of 128 keys) a masked call accepts:
 * 4096 tiles = 524288 keys.  A call with block_mask == NULL has no limit. */
#define BSA_MAX_KV_TILES 4096

typedef struct {
    int32_t batch;             /* B, number of sequences                        */
    int32_t total_q;           /* T, packed query tokens (= cu_seqlens_q[B])   */
    int32_t num_heads_q;       /* Hq                                            */
    int32_t num_heads_kv;      /* Hkv; Hq % Hkv == 0, 1 <= Hq/Hkv <= 16         */
    int32_t head_dim;          /* must be 128                                   */
    int32_t num_pages;         /* physical pages in kcache / vcache             */
    int32_t max_pages_per_seq; /* row length of block_table                     */
    int32_t max_seqlen_q;      /* upper bound of every Lq_b (sets the grid)    */
    int32_t mask_tiles_q;      /* block_mask dim 2 (max Q tiles per sequence)  */
    int32_t mask_tiles_kv;     /* block_mask dim 3 (KV tiles, Kb)              */
    int32_t kv_layout;         /* bsa_kv_layout                                 */
    int32_t causal;            /* 1: bottom-right causal; 0: no causal mask    */
    float softmax_scale;       /* >= 0 and finite, usually 1/sqrt(128); 0 gives
                                  uniform weights over each query's keys       */
} bsa_fp8_dims;

/*
 * bsa_fp8_prefill -- block-sparse FP8 attention prefill over a paged KV cache.
 *
 * q            E4M3 [T, Hq, 128], packed varlen queries (TND).
 * kcache,
 * vcache       E4M3 paged caches, layout dims->kv_layout, page_size slots
 *              per page.  Slots at or beyond Lkv_b may hold anything (NaN
 *              included): they never contribute.
 * qscale       float [T, Hq] Q descales (multiplied in).
 * kscale,
 * vscale       float, shapes per quant_type (see bsa_quant_type).
 * cu_seqlens_q int32 [B+1], leading 0, non-decreasing, ends at T.
 * block_table  int32 [B, max_pages_per_seq]: logical page -> physical page.
 *              Only entries of pages that hold keys < Lkv_b are read.
 * seqlens_kv   int32 [B], Lkv_b.  Query i of sequence b sits at position
 *              Lkv_b - Lq_b + i (bottom-right alignment); Lq_b > Lkv_b is
 *              allowed, and then, with the causal mask, the first
 *              Lq_b - Lkv_b queries see no key (O = 0, LSE = -FLT_MAX).
 * block_mask   uint8 [B, Hq, mask_tiles_q, mask_tiles_kv], non-zero = compute
 *              that (Q tile, KV tile) pair.  NULL = every tile (dense path).
 *              Bits above the causal range, at or beyond Lkv_b, or on Q tiles
 *              beyond Lq_b have no effect.
 * quant_type   bsa_quant_type.
 * page_size    32 or 64.
 * dims         sizes and flags (host pointer).
 * out          bf16 [T, Hq, 128] (TND), written for every query token.
 * lse          float [Hq, T], natural-log LSE; may be NULL (not written).
 * stream       hipStream_t to enqueue on.
 *
 * Preconditions the library cannot check (caller's contract):
 *   max_seqlen_q >= every Lq_b; with a mask,
 *   Lkv_b <= 128 * mask_tiles_kv (tiles beyond the mask width count as off);
 *   block_table entries of pages holding keys < Lkv_b are valid page ids;
 *   every descale is finite and >= 0.
 */
int bsa_fp8_prefill(const void* q, const void* kcache, const void* vcache,
                    const float* qscale, const float* kscale, const float* vscale,
                    const int32_t* cu_seqlens_q, const int32_t* block_table,
                    const int32_t* seqlens_kv, const uint8_t* block_mask,
                    int quant_type, int page_size, const bsa_fp8_dims* dims,
                    void* out, float* lse, void* stream);

/*
 * Options of the extended entry point.  A zero-initialised struct selects the
 * behaviour of bsa_fp8_prefill (TND queries, P-scale 256, block_mask form, no
 * schedule).
 *
 * q_layout        bsa_q_layout of q and qscale.  The output stays TND.
 * p_scale         Probability quantisation scale ("Quant Block Sparse
 *                 Attention", "Key parameters": p_scale).  Before the P.V
 *                 product each probability, taken against the running row
 *                 maximum, is multiplied by p_scale and rounded to E4M3; the
 *                 final normalisation divides the factor out again.  0 selects
 *                 256.  Values above 448 are rejected: the row maximum's
 *                 probability would then exceed the largest E4M3 value.
 * sparse_indices  Index-list form of the sparsity ("Quant Block Sparse
 * sparse_seq_len  Attention", "Sparse indices & PA page table"), device
 *                 pointers, both NULL or both set; block_mask must then be
 *                 NULL.  sparse_indices int32 [B, Hq, mask_tiles_q,
 *                 mask_tiles_kv] holds logical KV tile ids (tile n = keys
 *                 128n .. 128n+127); sparse_seq_len int32 [B, Hq,
 *                 mask_tiles_q] says how many leading entries of each row are
 *                 valid (clipped to 0 .. mask_tiles_kv).  Tiles are visited in
 *                 list order.  Entries that are negative, at or beyond
 *                 ceil(Lkv_b/128), or wholly above the causal range of the Q
 *                 tile select no keys and are skipped.  A tile id must not
 *                 repeat within a row (caller's contract).
 * qk_precision    bsa_qk_precision of the Q.K^T products.
 * schedule        NULL, or the task order written by bsa_fp8_schedule for the
 * schedule_len    same sparsity, sequence lengths and dims; schedule_len is
 *                 then the task count B * Hq * ceil(max_seqlen_q / 128).
 *                 The order changes which tasks run first, never a result:
 *                 every task is computed the same way whatever its position.
 */
typedef struct {
    int32_t q_layout;
    float p_scale;
    const int32_t* sparse_indices;
    const int32_t* sparse_seq_len;
    const int32_t* schedule;
    int32_t schedule_len;
    int32_t qk_precision;
} bsa_fp8_options;

/*
 * bsa_fp8_prefill_ex -- bsa_fp8_prefill with the options above ("Quant Block
 * Sparse Attention", "Key parameters": layout_q, p_scale, sparse_indices,
 * sparse_seq_len, metadata).  Arguments as for bsa_fp8_prefill; `options` is a
 * host pointer and may be NULL (= all defaults).  With the index-list form,
 * dims->mask_tiles_q and dims->mask_tiles_kv give the list shape (Qb, Kb) and
 * obey the same checks as the block_mask dimensions.  With q_layout NTD, q is
 * [Hq, T, 128] and qscale [Hq, T].
 */
int bsa_fp8_prefill_ex(const void* q, const void* kcache, const void* vcache,
                       const float* qscale, const float* kscale, const float* vscale,
                       const int32_t* cu_seqlens_q, const int32_t* block_table,
                       const int32_t* seqlens_kv, const uint8_t* block_mask,
                       int quant_type, int page_size, const bsa_fp8_dims* dims,
                       const bsa_fp8_options* options, void* out, float* lse,
                       void* stream);

/*
 * Scheduling pre-pass ("Quant Block Sparse Attention", "Sparse indices & PA
 * page table": the metadata that splits the (batch, query head, query block)
 * tasks between cores is produced on the device, on the same stream, and is
 * never read back by the host).
 *
 * A task is one (sequence b, q-head h, Q tile m) with id
 * (b * Hq + h) * ceil(max_seqlen_q / 128) + m.  Its cost is the number of KV
 * tiles the prefill visits for it: active tiles (mask bits, or valid list
 * entries) below ceil(Lkv_b/128) and inside the causal range, 0 for a Q tile
 * at or beyond Lq_b.  bsa_fp8_schedule writes every task id once into
 * `schedule`; entry i is the task that workgroup i of the prefill runs, and
 * the GPU hands workgroup i to XCD i mod 8 (each XCD has its own L2).  When
 * Hq is a multiple of 8, XCD x owns the q-heads [x*Hq/8, (x+1)*Hq/8) with all
 * their sequences and Q tiles; its tasks, sorted by decreasing cost (costs
 * above 1023 count as 1023), equal costs by increasing id, fill entries x,
 * x+8, x+16, ...  Otherwise all tasks, sorted the same way, fill the entries
 * in order.  Long tasks then start first and short ones fill the tail.
 *
 * bsa_fp8_schedule_workspace_bytes returns the size of the device workspace
 * the pass needs (0 for no tasks, -1 for invalid dims).  `workspace` must be a
 * device buffer of at least that many bytes, 16-byte aligned; its contents on
 * entry do not matter and on return are unspecified.  `schedule` is int32
 * [B * Hq * ceil(max_seqlen_q/128)].  block_mask, sparse_indices and
 * sparse_seq_len as for bsa_fp8_prefill_ex (all NULL = dense); `options` may
 * be NULL; only its sparse_indices / sparse_seq_len are read.  Four kernels are
 * enqueued on `stream`.  Errors as for bsa_fp8_prefill_ex, plus
 * BSA_ERR_NULL_POINTER when workspace or schedule is NULL with tasks present.
 */
long long bsa_fp8_schedule_workspace_bytes(const bsa_fp8_dims* dims);
int bsa_fp8_schedule(const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                     const uint8_t* block_mask, const bsa_fp8_dims* dims,
                     const bsa_fp8_options* options, void* workspace,
                     int32_t* schedule, void* stream);

/*
 * bsa_fp8_quantize_append -- produce the prefill's FP8 inputs from bfloat16
 * activations: quantise the query chunk and append its keys and values to the
 * paged cache.  Method (FlashMLA FP8 KV-cache article, "Quant/dequant
 * source"): a row of 128 values gets the descale d = amax/448 (amax = its
 * largest magnitude; scale_mode POW2 rounds d up to a power of two; a row of
 * zeros gets d = 1), and each value is stored as the E4M3 value of x/d,
 * rounded to nearest even and saturated at 448.  The divisions are IEEE
 * float32.  Which rows get a computed descale follows the quantisation
 * schemes of the prefill (bsa_quant_type):
 *   Q   always, per (token, head): q_out E4M3 [T, Hq, 128] (TND), qscale_out
 *       float [T, Hq];
 *   K   quant type 1: per (token, kv-head), descale written to kscale_cache at
 *       the row's (page, slot, kv-head) place; quant type 0: the given
 *       per-tensor descale kscale[0];
 *   V   the given descale: vscale[0] (type 0) or vscale[kv-head] (type 1).
 * Appending ("Quant Block Sparse Attention", "Key parameters" and "Sparse
 * indices & PA page table": paged cache, the query chunk at the tail of the
 * KV sequence): token i of sequence b's chunk (cu_seqlens_q) is stored at
 * logical position Lkv_b - Lq_b + i (seqlens_kv holds the lengths after the
 * append), i.e. page block_table[b, pos / page_size], slot pos % page_size,
 * in dims->kv_layout.  No other slot or descale is written.
 *
 * q_in         bf16 [T, Hq, 128], or NULL to skip the queries (q_out and
 *              qscale_out may then be NULL).
 * k_in, v_in   bf16 [T, Hkv, 128], both NULL to skip the append.
 * dims         batch, total_q (T), num_heads_q, num_heads_kv, head_dim,
 *              max_pages_per_seq, kv_layout are read; the other fields must be
 *              valid as for bsa_fp8_prefill (their values are not used).
 * Every array is a device pointer owned by the caller; one kernel is enqueued
 * on `stream`.  Preconditions: Lq_b <= Lkv_b (every appended position is at
 * least 0; the prefill itself also accepts Lq_b > Lkv_b), valid block-table
 * entries for the appended positions, finite inputs, positive given
 * descales.  Errors: as for bsa_fp8_prefill, plus BSA_ERR_SCALE_MODE;
 * BSA_ERR_NULL_POINTER when a pointer the requested parts need is NULL or
 * only one of k_in / v_in is given.
 */
int bsa_fp8_quantize_append(const void* q_in, const void* k_in, const void* v_in,
                            const int32_t* cu_seqlens_q, const int32_t* seqlens_kv,
                            const int32_t* block_table, const float* kscale, const float* vscale,
                            int quant_type, int page_size, int scale_mode, const bsa_fp8_dims* dims,
                            void* q_out, float* qscale_out, void* kcache, void* vcache,
                            float* kscale_cache, void* stream);

/*
 * FP8 sparse decode (the workload of the FlashMLA FP8 sparse decoding article:
 * section "FP8 KVCache format" and its description of the MQA decode step).
 *
 * Multi-query attention: every query head reads the same single KV head.  A
 * cache row (one token) is 656 bytes: 512 E4M3 codes (key dims 0..511, four
 * 1x128 tiles), 4 float32 descales (one per tile), 64 bfloat16 values (key
 * dims 512..575).  Dequantised key k^ = code * descale (dims 0..511) and the
 * bfloat16 values (dims 512..575); the value is v^ = k^[0..511].  Each entry of
 * an index list names one cache row as page-block index * page_size + offset
 * within the block, and -1 marks an unused entry (the article's
 * quick-reproduce paragraph: indices of shape (batch, seq_len_q, topk) passed
 * as indices_in_kvcache).  Entry e is therefore the row at page e / page_size,
 * slot e % page_size.  For query token (b, s) and head h:
 *   Omega   = the entries of indices[b, s, :] inside [0, num_pages * page_size)
 *             (any other entry, -1 included, selects nothing; an entry listed
 *             twice counts twice)
 *   score_j = softmax_scale * q[b, s, h, :] . k^_j      (576 dims)
 *   out[b, s, h, :] = sum_{j in Omega} softmax_j(score) v^_j
 *   lse[b, h, s]    = ln sum_{j in Omega} exp(score_j)
 * An empty Omega gives out = 0 and lse = -FLT_MAX ("Quant Block Sparse
 * Attention", "Sparse indices & PA page table": the empty-task convention).
 * No block table or sequence length enters: the lists address cache rows
 * directly, so a caller that tracks token positions converts them with its
 * own block table (row = block_table[b][pos / page_size] * page_size +
 * pos % page_size).  Dequantised values are rounded to bfloat16 and P to
 * bfloat16 before the bfloat16 matrix products, as the article's kernel does;
 * with power-of-two descales (its reference quantiser) the dequantisation is
 * exact.
 */
typedef struct {
    int32_t batch;             /* B                                             */
    int32_t s_q;               /* query tokens per sequence                     */
    int32_t num_heads_q;       /* h_q, a multiple of 64                         */
    int32_t topk;              /* entries per index list, >= 1                  */
    int32_t num_pages;         /* pages of kv_cache                             */
    int32_t page_size;         /* slots per page, >= 1                          */
    float softmax_scale;       /* finite                                        */
} bsa_fp8_decode_dims;

/*
 * q           bf16 [B, s_q, h_q, 576]
 * kv_cache    uint8 [num_pages, page_size, 656]
 * indices     int32 [B, s_q, topk], cache rows page * page_size + slot (any
 *             order; -1 = unused)
 * out         bf16 [B, s_q, h_q, 512]; lse float [B, h_q, s_q] or NULL
 * Device pointers owned by the caller; one kernel on `stream`; nothing is
 * allocated.  Errors: BSA_ERR_NULL_POINTER, BSA_ERR_SIZE (negative sizes,
 * topk < 1), BSA_ERR_GQA (h_q not a multiple of 64), BSA_ERR_PAGE_SIZE
 * (page_size < 1), BSA_ERR_SOFTMAX_SCALE (not finite), BSA_ERR_TOO_LARGE
 * (topk above BSA_DECODE_MAX_TOPK, grid or num_pages * page_size past 2^31),
 * BSA_ERR_LAUNCH.  Rows no entry names are never read, so they may hold
 * anything.  Equivalent to bsa_fp8_sparse_decode_ex with num_splits = 1.
 */
#define BSA_DECODE_MAX_TOPK 8192   /* longest index list one workgroup holds      */
#define BSA_DECODE_MAX_SPLITS 256
int bsa_fp8_sparse_decode(const void* q, const void* kv_cache, const int32_t* indices,
                          const bsa_fp8_decode_dims* dims, void* out, float* lse, void* stream);

/*
 * Split-list sparse decode: the same result as bsa_fp8_sparse_decode, with
 * each index list cut into num_splits contiguous parts that separate
 * workgroups attend to, and a second kernel that merges the parts.  This is
 * the decode kernel's way of occupying the chip when B * s_q is small (the
 * FlashMLA FP8 sparse decoding article: its launch grid carries a dimension
 * of "SM parts" beside the heads and s_q, and its decode loop is preceded by
 * a scheduling-metadata call); it also admits lists longer than
 * BSA_DECODE_MAX_TOPK (the article quotes runs at topk 16384 and 32768).
 *
 * Part p covers list entries [p*E, (p+1)*E) with E = 32 * ceil(ceil(topk/32) /
 * num_splits); a part may be empty.  For each (b, s, h) part p stores
 * O_p = its own softmax-weighted value sum and lse_p (log2 domain, -inf when
 * it selects nothing) in the workspace; the merge with M = max_p lse_p and
 * w_p = 2^(lse_p - M) writes out = sum_p w_p O_p / sum_p w_p and
 * lse = ln 2 * (M + log2 sum_p w_p), or out = 0 and lse = -FLT_MAX when every
 * part is empty.  This is exactly the single-pass softmax regrouped; only the
 * rounding differs.
 *
 * num_splits  1 .. BSA_DECODE_MAX_SPLITS; ceil(ceil(topk/32) / num_splits) * 32
 *             must not exceed BSA_DECODE_MAX_TOPK
 * workspace   device memory of bsa_fp8_sparse_decode_workspace_bytes(dims,
 *             num_splits) bytes, 16-byte aligned, owned by the caller and
 *             overwritten (NULL allowed when num_splits == 1); calls that share
 *             a workspace must be ordered on one stream
 * Other arguments as for bsa_fp8_sparse_decode.  Two kernels on `stream`
 * (one when num_splits == 1); nothing is allocated.  Errors: as for
 * bsa_fp8_sparse_decode, plus BSA_ERR_SIZE (num_splits out of range, a
 * workspace not 16-byte aligned), BSA_ERR_NULL_POINTER (workspace NULL with
 * num_splits > 1), BSA_ERR_TOO_LARGE (a part longer than BSA_DECODE_MAX_TOPK,
 * or B * s_q * h_q past 2^31 with num_splits > 1).
 */
int bsa_fp8_sparse_decode_ex(const void* q, const void* kv_cache, const int32_t* indices,
                             const bsa_fp8_decode_dims* dims, int num_splits, void* workspace,
                             void* out, float* lse, void* stream);

/*
 * bsa_fp8_sparse_decode_noalloc -- bsa_fp8_sparse_decode_ex for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * and harnesses that forbid hipMalloc.  The partial results live in a static
 * device array of the library (BSA_DECODE_SCRATCH_BYTES, one per GPU, held
 * until the process ends) instead of a caller workspace; nothing is
 * allocated and no allocating routine is called.  The caller still passes q,
 * kv_cache, indices, out and lse.
 *
 * num_splits  0 = the part count of bsa_fp8_sparse_decode_num_splits, lowered
 *             until the partial results fit the scratch; else 1 ..
 *             BSA_DECODE_MAX_SPLITS as for bsa_fp8_sparse_decode_ex.
 * Errors: as for bsa_fp8_sparse_decode_ex, plus BSA_ERR_SCRATCH when
 * num_splits * B * s_q * h_q * 513 * 4 bytes exceed BSA_DECODE_SCRATCH_BYTES
 * (checked before any HIP call), and BSA_ERR_LAUNCH when the scratch's device
 * address cannot be obtained.  All calls on one GPU share its scratch: calls
 * that may run at the same time on one GPU (on different streams, or from
 * different threads) race and must be ordered by the caller.  The first call
 * on a device looks up the scratch's address there, with that device current.
 */
#define BSA_DECODE_SCRATCH_BYTES (64 * 1024 * 1024)
int bsa_fp8_sparse_decode_noalloc(const void* q, const void* kv_cache, const int32_t* indices,
                                  const bsa_fp8_decode_dims* dims, int num_splits, void* out,
                                  float* lse, void* stream);

/*
 * Workspace bytes bsa_fp8_sparse_decode_ex needs: 0 for num_splits == 1,
 * else num_splits * B * s_q * h_q * 513 * 4 (float32 partial outputs and
 * log-sum-exps).  -1 for NULL dims, negative sizes or num_splits out of range.
 */
long long bsa_fp8_sparse_decode_workspace_bytes(const bsa_fp8_decode_dims* dims, int num_splits);

/*
 * A part count for bsa_fp8_sparse_decode_ex (host only, no device access): the
 * fewest parts whose row lists fit (at most BSA_DECODE_MAX_TOPK entries each),
 * raised until the decode grid has about 256 workgroups (one per compute
 * unit) but never below 2 blocks of 32 entries per part, capped at
 * BSA_DECODE_MAX_SPLITS.  1 for NULL dims or dims the decode rejects.
 */
int bsa_fp8_sparse_decode_num_splits(const bsa_fp8_decode_dims* dims);

/* Static text for a bsa_status value (never NULL). */
const char* bsa_fp8_status_string(int status);

/* Library ABI version, currently 4. */
int bsa_fp8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_FP8_H */
