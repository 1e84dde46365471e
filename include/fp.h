/*
 * fp.h - C ABI of the ForwardPass attention step on a paged KV pool (MI355X / gfx950).
 *
 * One pass carries several lanes (independent sequences) whose rows are
 * concatenated and addressed by a row-offset array `indptr`, all run in one
 * launch per stage (Pie docs, "The forward pass", section Lanes). Its
 * StateGeometry gives, per row, a RoPE position and the working-set slot the
 * row writes, and per lane, how many slots attention reads (kv_len) and how
 * many newly written slots to freeze afterwards (fold) (section State
 * geometry, field table). A lane may carry a per-row slot bitmap instead of
 * the causal rule (section Attention masks); the caller picks readout rows
 * (section Readouts). KV state is paged (Pie reviews, section 2.1/2.2,
 * Eqs. (1) and (2)); the pages of a lane's working set are listed in slot order.
 *
 * A step is four calls, enqueued in this order on one stream:
 *   fp_append_kv -> fp_attend -> fp_fold -> fp_readout
 * (or three, with fp_fold_readout in place of the last two).
 * A repeating decode loop may enqueue fp_advance after fp_fold to write the
 * next pass's geometry on the device.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the name ends in `_host`.
 *  - bf16 values are passed as 16-bit storage (bit patterns). The pool, Q, K
 *    and V arrays and fp_attend's `out` must be 16-byte aligned
 *    (FP_ERR_UNSUPPORTED otherwise): the kernels move them in 16-byte vectors.
 *  - The caller owns every buffer; the library allocates no memory, keeps no
 *    state between calls (apart from the static device scratch of
 *    fp_attend_noalloc) and never synchronizes. Buffers must stay valid until
 *    the work enqueued on `stream` has completed. `stream` may be NULL (the
 *    default stream).
 *  - Errors the host can see are returned synchronously, before anything is
 *    enqueued (FP_ERR_*). Errors that depend on device data never stop the
 *    stream: the kernel ORs a bit into *status (an int32 the caller zeroes)
 *    and suppresses or clamps the offending access (FP_ST_*).
 *  - Calls that overlap on one stream run in order (like passes on a Pie
 *    Pipeline); two streams writing the same pool pages race.
 */
#ifndef FP_H_
#define FP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;   /* same opaque types as HIP's */
typedef struct ihipEvent_t *hipEvent_t;

/* ---- return codes (host-detected, nothing enqueued) ---- */
#define FP_OK               0
#define FP_ERR_NULL        (-1)   /* a required pointer is NULL                              */
#define FP_ERR_SHAPE       (-2)   /* inconsistent sizes (e.g. H_q % H_kv != 0, num_lanes < 1) */
#define FP_ERR_UNSUPPORTED (-3)   /* head_dim not 64/128, page_size not 8/16/32, ...          */
#define FP_ERR_WORKSPACE   (-4)   /* workspace smaller than fp_attend_workspace_bytes()       */
#define FP_ERR_HIP         (-5)   /* a HIP launch failed                                      */

/* ---- device status bits (ORed into *status) ---- */
#define FP_ST_SLOT_RANGE     1    /* row slot outside [0, capacity): its write suppressed     */
#define FP_ST_FROZEN         2    /* row slot below committed_len: its write suppressed      */
#define FP_ST_KVLEN          4    /* kv_len outside [0, capacity]: clamped                    */
#define FP_ST_FOLD_CLAMP     8    /* fold count outside [0, rows of lane]: clamped            */
#define FP_ST_READOUT_RANGE 16    /* readout row outside [0, num_rows): zero row written      */
#define FP_ST_MASK_SHORT    32    /* mask row has fewer than kv_len bits: missing bits are 0  */
#define FP_ST_PAGE_RANGE    64    /* page id outside [0, num_pages): write suppressed, read clamped */
#define FP_ST_PLAN_MISMATCH 128   /* device offset arrays disagree with their host copies:
                                     fp_attend did no attention work (outputs untouched)      */
#define FP_ST_ADAPTER      256    /* adapter id >= num_adapters: the lane's rows keep y       */
#define FP_ST_DUP_WRITE    512    /* fp_check_hazards: a KV cell is written twice in one pass */
#define FP_ST_SHARED_CELL 1024    /* fp_check_hazards: a KV cell one lane writes is read or
                                     written by another lane (Eq. (4) violated)               */

/* ---- fold sentinels (StateGeometry.fold; a value >= 0 is a literal count) ---- */
#define FP_FOLD_ALL      (-1)     /* freeze every row written this pass                       */
#define FP_FOLD_CHANNEL  (-2)     /* freeze channel[lane] rows, a count written on the device */

/*
 * StateGeometry of one pass (Pie docs, "The forward pass", State geometry).
 * Rows of lane l are [indptr[l], indptr[l+1]).
 */
typedef struct fp_geometry {
    int32_t num_lanes;           /* L >= 1                                                    */
    int32_t num_rows;            /* N = indptr[L]                                             */
    const int32_t *indptr;       /* [L+1] row offsets, non-decreasing, indptr[0] = 0          */
    const int32_t *indptr_host;  /* [L+1] host copy of indptr: used to size launches only     */
    const int32_t *positions;    /* [N] RoPE position id of each row                          */
    const int32_t *slots;        /* [N] working-set slot each row writes                      */
    const int32_t *kv_len;       /* [L] slots each lane reads this pass                       */
    const int32_t *fold;         /* [L] literal count >= 0, FP_FOLD_ALL or FP_FOLD_CHANNEL    */
} fp_geometry;

/*
 * One attention layer of the paged KV pool.
 *
 * Page layout (bf16, page p at element offset p * 2*H*P*d):
 *     K block  [H][P][d]   K[h][o][:] is slot o of the page, rotated by RoPE
 *     V block  [H][d][P]   V stored transposed: V[h][:][o] is slot o
 * Slot s of lane l lives in page page_ids[page_indptr[l] + s / P] at offset
 * s % P. Lane l's capacity is (page_indptr[l+1] - page_indptr[l]) * P slots.
 * Pages may be shared read-only between lanes; a page written this pass must
 * belong to exactly one lane.
 */
typedef struct fp_kv_pool {
    void *kv;                        /* bf16 pages, num_pages * 2*H*P*d elements             */
    int32_t num_pages;
    int32_t page_size;               /* P in {8, 16, 32}                                      */
    int32_t num_kv_heads;            /* H                                                     */
    int32_t head_dim;                /* d in {64, 128}                                        */
    const int32_t *page_indptr;      /* [L+1] offsets into page_ids                           */
    const int32_t *page_indptr_host; /* [L+1] host copy: used to size launches only           */
    const int32_t *page_ids;         /* [page_indptr[L]] physical page of each working-set page */
    int32_t *committed_len;          /* [L] frozen slots per lane; fp_fold adds to it         */
} fp_kv_pool;

/*
 * Per-row slot bitmaps (Pie docs, "The forward pass", Attention masks).
 * Lane l's words are bits[word_offset[l] .. word_offset[l+1]); an empty span
 * means the lane keeps the causal rule. A non-empty span holds, for each of
 * the lane's rows in order, the same number of uint32 words (span / rows);
 * bit b of word w (LSB first) says the row attends slot 32*w + b. The bitmap
 * replaces the causal rule for its lane; bits at or beyond kv_len are ignored.
 */
typedef struct fp_mask {
    const uint32_t *bits;
    const int64_t *word_offset;       /* [L+1]                                                */
    const int64_t *word_offset_host;  /* [L+1] host copy: used to size launches only          */
} fp_mask;

/*
 * Optional tuning and profiling hooks for fp_attend; pass NULL for defaults.
 * Results do not depend on it beyond fp rounding order.
 */
typedef struct fp_tuning {
    int32_t decode_split_slots;       /* KV slots per decode work item, multiple of 32; 0: the
                                         largest of 4096/2048/1024/512 that gives each resident
                                         decode workgroup of the device about two items      */
    int32_t reserved[7];              /* must be zero                                          */
    hipEvent_t attn_begin;            /* nullable: recorded on the stream right before the
                                         attention kernels (prefill, then decode)             */
    hipEvent_t attn_end;              /* nullable: recorded right after them (before the merge of
                                         decode splits)                                       */
    hipEvent_t prefill_end;           /* nullable: recorded between the prefill and the decode
                                         kernels (right after attn_begin if no prefill lane)  */
    hipEvent_t merge_end;             /* nullable: recorded after the merge of decode splits
                                         (right after attn_end if nothing is merged)          */
} fp_tuning;

/*
 * fp_append_kv - write each row's K (RoPE-rotated at positions[r]) and V into
 * slot slots[r] of its lane's working set (State geometry: positions, slots;
 * folding appends rows causally).
 *   k, v : bf16 [N][H][d], un-rotated K and V of the pass's rows.
 *   RoPE : pairs (2i, 2i+1) rotated by positions[r] * rope_theta^(-2i/d),
 *          computed in fp64 and rounded once to bf16.
 * A write whose slot is outside the lane's capacity (FP_ST_SLOT_RANGE) or below
 * committed_len (FP_ST_FROZEN) is suppressed. Two rows of one pass writing the
 * same slot of one lane is undefined.
 */
int fp_append_kv(const fp_kv_pool *pool, const fp_geometry *geom, const void *k, const void *v,
                 float rope_theta, int32_t *status, hipStream_t stream);

/* Workspace bytes fp_attend needs for this geometry (host-only, reads *_host arrays). */
int64_t fp_attend_workspace_bytes(const fp_kv_pool *pool, const fp_geometry *geom, const fp_mask *mask,
                                  int32_t num_q_heads, const fp_tuning *tuning);

/*
 * fp_attend - softmax attention of every row over its lane's first kv_len
 * slots (State geometry: kv_len; Attention masks).
 *   q   : bf16 [N][H_q][d], un-rotated; rotated at positions[r] like K.
 *   rule: without a bitmap, row r reads slots j <= slots[r] (j < kv_len);
 *         with one, the slots whose bits are set (j < kv_len).
 *   GQA : query head q reads KV head q / (H_q / H_kv).
 *   out : fp32 [N][H_q][d]; lse: fp32 [N][H_q] natural-log sum-exp (nullable).
 *         A row with no readable slot gets out = 0 and lse = -inf.
 *   sm_scale multiplies q.k (use 1/sqrt(d) for the usual scaling).
 *   mask may be NULL (every lane causal).
 * Slots at or beyond kv_len are never read, whatever they hold.
 */
int fp_attend(const fp_kv_pool *pool, const fp_geometry *geom, const void *q, int32_t num_q_heads,
              float rope_theta, float sm_scale, const fp_mask *mask, float *out, float *lse,
              void *workspace, size_t workspace_bytes, const fp_tuning *tuning,
              int32_t *status, hipStream_t stream);

/*
 * fp_attend_noalloc - fp_attend for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results as fp_attend, but
 * the workspace is the library's own static device scratch of
 * fp_attend_noalloc_max_bytes() bytes (64 MiB) per device, which every device
 * the library runs on holds until the process ends. The caller still passes
 * inputs and outputs.
 *   - Makes no hipMalloc / hipFree call and calls no allocating routine. The
 *     first call on a device looks up that device's scratch address once
 *     (hipGetSymbolAddress); make that first call outside graph capture.
 *   - Returns FP_ERR_WORKSPACE, with nothing enqueued, when the pass needs more
 *     than the scratch holds (fp_attend_workspace_bytes() > the maximum), and
 *     the other FP_ERR_* codes of fp_attend.
 *   - Every call on one device shares that device's scratch, which keeps the
 *     last call's contents (nothing in it needs to start at zero). Calls that
 *     overlap on one device (two streams, or two host threads without ordering)
 *     race on it; calls in order on one stream do not. fp_attn_mass cannot follow
 *     it (that needs the rotated queries in a caller workspace).
 */
int fp_attend_noalloc(const fp_kv_pool *pool, const fp_geometry *geom, const void *q, int32_t num_q_heads,
                      float rope_theta, float sm_scale, const fp_mask *mask, float *out, float *lse,
                      const fp_tuning *tuning, int32_t *status, hipStream_t stream);

/* Bytes of the static scratch fp_attend_noalloc uses (the largest workspace it accepts). */
int64_t fp_attend_noalloc_max_bytes(void);

/*
 * fp_fold - after the pass, freeze k_l newly written slots of every lane:
 * committed_len[l] += k_l, where k_l = fold[l] (literal), the lane's row count
 * (FP_FOLD_ALL) or channel[l] (FP_FOLD_CHANNEL, a count another kernel wrote on
 * the device, read without a host round trip). Counts are clamped to
 * [0, rows of lane] (FP_ST_FOLD_CLAMP). channel may be NULL if no lane uses it
 * (a lane that does then folds 0 and sets FP_ST_FOLD_CLAMP).
 * (State geometry: fold; speculative-decoding paragraph.)
 */
int fp_fold(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *channel,
            int32_t *status, hipStream_t stream);

/*
 * fp_readout - gather readout rows of `out` (Readouts section).
 *   rows == NULL : the last row of every lane with at least one row, in lane
 *                  order; num_readout must equal the number of such lanes.
 *   rows != NULL : rows[0..num_readout) are global row indices, copied in the
 *                  given order; an index outside [0, N) gives a zero row and
 *                  FP_ST_READOUT_RANGE.
 *   dst : fp32 [num_readout][row_elems], row_elems = H_q * d.
 */
int fp_readout(const fp_geometry *geom, const float *out, int32_t row_elems, const int32_t *rows,
               int32_t num_readout, float *dst, int32_t *status, hipStream_t stream);

/*
 * fp_fold_readout - fp_fold and fp_readout of the same pass in one launch (the
 * two stages read and write disjoint memory, so neither waits on the other).
 * Arguments, results and status bits are exactly those of
 * fp_fold(pool, geom, channel, status) followed by
 * fp_readout(geom, out, row_elems, rows, num_readout, dst, status). Every
 * check of both calls runs before anything is enqueued: on an error neither
 * stage runs.
 */
int fp_fold_readout(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *channel, const float *out,
                    int32_t row_elems, const int32_t *rows, int32_t num_readout, float *dst, int32_t *status,
                    hipStream_t stream);

/* Workspace bytes fp_check_hazards needs: three int32 per KV cell (num_pages * P cells). */
int64_t fp_hazard_workspace_bytes(const fp_kv_pool *pool);

/*
 * fp_check_hazards - debug check of one pass's geometry against the reviews'
 * Eq. (4) (section 5: calls batched together must keep their meaning, i.e.
 * W(a) ∩ (R(b) ∪ W(b)) = ∅ for two calls a ≠ b), with lanes as the calls and
 * KV cells (physical page, offset) as the state:
 *   W(l) = cells lane l's rows write (the writes fp_append_kv performs: slot
 *          inside the capacity, not below committed_len, page id in the pool);
 *   R(l) = cells of lane l's slots below its kv_len (clamped to the capacity)
 *          whose page id is in the pool.
 * Sets FP_ST_DUP_WRITE in *status if some cell is written more than once in
 * the pass (two rows naming one slot, which fp_append_kv leaves undefined, or
 * two lanes whose pages overlap), and FP_ST_SHARED_CELL if a cell one lane
 * writes is read or written by another lane. Reads the geometry, the page
 * table and committed_len only: enqueue it before fp_append_kv of the pass.
 *   workspace: fp_hazard_workspace_bytes(pool) bytes of device memory (its
 *   contents are overwritten). Four launches; nothing else is modified.
 * Returns FP_ERR_NULL / FP_ERR_SHAPE / FP_ERR_UNSUPPORTED / FP_ERR_WORKSPACE
 * before enqueueing anything, FP_ERR_HIP on a launch error.
 */
int fp_check_hazards(const fp_kv_pool *pool, const fp_geometry *geom, void *workspace, size_t workspace_bytes,
                     int32_t *status, hipStream_t stream);

/*
 * fp_attn_mass - attention statistics of the pass, so that an eviction policy
 * driven by attention scores (TOVA and the like) can run on the device: the
 * pages' review (section 7) notes that such a policy needs the forward pass to
 * return the scores, and the Docs' Attention masks section names score-based
 * KV eviction among the uses of per-row masks. For lane l, KV head g and slot
 * j below the lane's kv_len (clamped to its capacity):
 *   slot_mass[g * S + page_indptr[l] * P + j] +=
 *       sum over the lane's rows r and the query heads h of KV head g of
 *       exp(score(r, h, j) - lse[r][h])   if row r may read slot j, else 0,
 * with S = page_indptr_host[L] * P and score the scaled q.k of fp_attend. Each
 * row's probabilities sum to one over its readable slots, so summed over all
 * slots and KV heads the pass adds the count of (row, query head) pairs that
 * read at least one slot.
 *   Call after fp_attend on the same stream with the same pool, geom,
 *   num_q_heads, mask and workspace: it reads the rotated queries that
 *   fp_attend left at the start of the workspace and fp_attend's lse output
 *   (non-null); tuning may differ from fp_attend's (it is only validated).
 *   The workspace must hold at least the rotated queries, N * H_q * d * 2 bytes.
 *   slot_mass: fp32 [H_kv][S] device, accumulated into (zero it for the mass of
 *   one pass); entries of slots at or past kv_len are not touched.
 * Deterministic: every output word has one writer and a fixed summation order.
 * Returns FP_ERR_NULL / FP_ERR_SHAPE / FP_ERR_WORKSPACE like fp_attend.
 */
int fp_attn_mass(const fp_kv_pool *pool, const fp_geometry *geom, int32_t num_q_heads, const fp_mask *mask,
                 const float *lse, const void *workspace, size_t workspace_bytes, const fp_tuning *tuning,
                 float *slot_mass, hipStream_t stream);

/*
 * fp_tova_mask - score-driven KV eviction on the device: the next pass's
 * per-row bitmaps from the attention mass of earlier passes. The Docs'
 * Attention masks section names attention-based eviction such as TOVA among
 * the uses of per-row masks, and the review's section 7 has the forward pass
 * return the scores it needs (fp_attn_mass); the policy itself is not spelled
 * out there, and this call takes the following reading of it.
 *   For the pass given by pool and geom (call it before that pass's
 *   fp_append_kv: committed_len must still be the frozen length), lane l's old
 *   slots are j < c_l = committed_len[l] (clamped to the lane's capacity), and
 *     score_l(j) = sum over KV heads g = 0 .. H-1, in that order, in fp32, of
 *                  slot_mass[g * S + page_indptr[l] * P + j],  S = page_indptr_host[L] * P.
 *   Old slot j is a candidate unless prev_keep is given, j < prev_limit[l]
 *   (clamped to [0, c_l]) and bit j of the lane's prev_keep words is clear:
 *   a slot dropped by an earlier selection stays dropped. The lane keeps the
 *   min(max(budget[l], 0), #candidates) candidates with the largest score,
 *   scores compared as the total order of fp32 bit patterns (negatives below
 *   positives), equal scores going to the lower slot.
 *   keep: written, lane l's words at keep[keep_word_offset[l] ..]: the first
 *     ceil(c_l / 32) words, bit j set iff old slot j is kept. keep_word_offset
 *     (int64 [L+1], device) must give every lane at least ceil(capacity / 32)
 *     words, the same layout as prev_keep; keep must not overlap prev_keep.
 *   mask_bits / mask_word_offset: the pass's bitmaps (fp_mask layout), written
 *     for every lane with a non-empty span: row r of lane l, word w < span / rows,
 *     bit j = 32w + b is set iff j < kv_len[l] (clamped to capacity) and
 *       j <  c_l : old slot j is kept;
 *       j >= c_l : j <= slots[r] (the pass's own slots, by the slot-order rule).
 *     A span with fewer than ceil(kv_len / 32) words per row sets
 *     FP_ST_MASK_SHORT. Lanes with an empty span keep the causal rule; their
 *     keep words are still written.
 * Deterministic (exact integer selection; every output word has one writer).
 * Returns FP_ERR_NULL / FP_ERR_SHAPE like fp_attend.
 */
int fp_tova_mask(const fp_kv_pool *pool, const fp_geometry *geom, const float *slot_mass, const int32_t *budget,
                 const uint32_t *prev_keep, const int32_t *prev_limit, const int64_t *keep_word_offset,
                 uint32_t *keep, uint32_t *mask_bits, const int64_t *mask_word_offset,
                 const int64_t *mask_word_offset_host, int32_t *status, hipStream_t stream);

/*
 * fp_advance - the StateGeometry of the next pass of a repeating decode loop,
 * written on the device from committed_len, so a loop that keeps its decode
 * pass in flight (Pipelines and frames: run_ahead) never waits on the host for
 * the lengths a fold produced (State geometry: folding appends rows causally
 * after the frozen prefix; speculative decoding rewinds to the accepted prefix
 * this way). For lane l with n_l = indptr[l+1] - indptr[l] rows (the shape of
 * the next pass, fixed by the caller) and c_l = committed_len[l]:
 *   slots[indptr[l] + i]     = c_l + i                               i < n_l
 *   positions[indptr[l] + i] = c_l + i + (pos_offset ? pos_offset[l] : 0)
 *   kv_len[l]                = c_l + n_l
 *   geom      : the next pass's geometry; indptr / indptr_host / num_lanes /
 *               num_rows are read, positions / slots / kv_len are the device
 *               arrays written (geom->positions etc. are ignored: the writable
 *               outputs are the arguments below), fold is untouched.
 *   pos_offset: nullable int32 [L] device, position of slot 0 of each lane.
 *   positions, slots : int32 [N] device outputs; kv_len : int32 [L] device output.
 * Enqueue after fp_fold of the previous pass on the same stream. Nothing is
 * validated on the device here: a slot past the lane's pages is caught by
 * fp_append_kv (FP_ST_SLOT_RANGE) and kv_len by fp_attend (FP_ST_KVLEN).
 * Returns FP_ERR_NULL / FP_ERR_SHAPE for bad arguments, FP_ERR_HIP on a launch error.
 */
int fp_advance(const fp_kv_pool *pool, const fp_geometry *geom, const int32_t *pos_offset, int32_t *positions,
               int32_t *slots, int32_t *kv_len, hipStream_t stream);

/*
 * Projection-site LoRA adapters (Docs, section Adapters: an adapter attached
 * at a projection site maps the projection input x and the base output y to
 * y + b * (a * x), and requests in one batch may use different adapters).
 * Adapter k is A_k (rank x d_in), B_k (d_out x rank) and a scale s_k.
 */
typedef struct fp_lora {
    int32_t num_adapters;             /* >= 1                                                   */
    int32_t rank;                     /* r in {16, 32, 48, 64}                                  */
    int32_t d_in, d_out;              /* projection widths: d_in a multiple of 64, d_out a       */
                                      /* multiple of 32 and at most 65535 * 512                  */
    const void *a;                    /* bf16 [num_adapters][rank][d_in] device                 */
    const void *b;                    /* bf16 [num_adapters][d_out][rank] device                */
    const float *scale;               /* [num_adapters] device                                  */
} fp_lora;

/* Workspace bytes fp_adapter_lora needs (host-only): the rank-r projections of every row (two bf16 terms),
 * then 16 bytes per (lane, 32-row block) work item. */
int64_t fp_lora_workspace_bytes(const fp_geometry *geom, const fp_lora *lora);

/*
 * fp_adapter_lora - for every row r of lane l with k = adapter[l] >= 0:
 *     out[r] = bf16( y[r] + s_k * B_k (A_k x[r]) )
 * and out[r] = y[r] for lanes with adapter[l] < 0.
 *   geom   : only indptr / indptr_host / num_lanes / num_rows are read.
 *   adapter: int32 [L] device, per-lane adapter id; an id >= num_adapters sets
 *            FP_ST_ADAPTER and the lane keeps y.
 *   x      : bf16 [N][d_in]; y, out: bf16 [N][d_out]; out may equal y (in place).
 *   Arithmetic: v = A_k x in fp32 (MFMA), kept as two bf16 terms (hi + lo,
 *   16 significant bits), B_k v in fp32, then y + s_k * (B_k v) in fp32
 *   rounded to bf16.
 * Feeding a2: run it on the Q, K or V projection outputs before fp_append_kv /
 * fp_attend. Returns FP_ERR_NULL / FP_ERR_SHAPE / FP_ERR_UNSUPPORTED /
 * FP_ERR_WORKSPACE before enqueueing anything.
 */
int fp_adapter_lora(const fp_geometry *geom, const fp_lora *lora, const int32_t *adapter, const void *x,
                    const void *y, void *out, void *workspace, size_t workspace_bytes, int32_t *status,
                    hipStream_t stream);

/*
 * fp_adapter_ia3 - the IA3 form of a projection-site adapter (Docs, section
 * Adapters: IA3 scales the base output y): for every row r of lane l with
 * k = adapter[l] >= 0,
 *     out[r][c] = bf16( y[r][c] * scale_k[c] )
 * and out[r] = y[r] for lanes with adapter[l] < 0 (an id >= num_adapters sets
 * FP_ST_ADAPTER and keeps y). The product of two bf16 values is exact in fp32,
 * so the result is the correctly rounded product.
 *   scale  : bf16 [num_adapters][d_out] device; y, out: bf16 [N][d_out] (out may equal y);
 *   d_out a multiple of 8. geom: only indptr / indptr_host / num_lanes / num_rows are read.
 */
int fp_adapter_ia3(const fp_geometry *geom, int32_t num_adapters, int32_t d_out, const void *scale,
                   const int32_t *adapter, const void *y, void *out, int32_t *status, hipStream_t stream);

/*
 * fp_vertical_merge - vertical batching of a frame (the reviews' section 5:
 * a prefix forward and its continuation can be combined into one dispatch
 * when their order is preserved inside it; Docs, Pipelines and frames:
 * submit_frame runs passes back to back). Host-only: from the host copies of
 * two consecutive passes A then B over the same lanes and pool, decide
 * whether one pass M does exactly what A then B do, and if so describe M.
 *
 * Eligible when, for every lane l with c = committed[l] (before A), nA / nB
 * rows in A / B and capacity cap = (page_indptr_host[l+1] -
 * page_indptr_host[l]) * page_size:
 *   - A's rows take slots c, c+1, ..., c+nA-1 in order (rows appended
 *     causally after the frozen prefix), and A folds all of them (FP_FOLD_ALL
 *     or the literal nA), so B's rows see them as frozen history;
 *   - every B slot is >= c + nA (B never rewrites what A froze);
 *   - A's and B's kv_len lie in [0, cap], A's covers its rows (>= c + nA) and,
 *     when B has rows, so does B's (the merged pass reads B's kv_len);
 *   - B folds all its rows or a literal count in [0, nB];
 *   - no lane carries a mask (the caller passes passes without bitmaps).
 * Then M has, per lane, A's rows followed by B's, kv_len = B's (A's if B has
 * no rows), and fold = FP_FOLD_ALL if B folds all, else the literal nA + k.
 * Under the causal rule an A row reads j <= its slot, none of B's slots, and a
 * B row reads A's slots as freshly appended K/V: the same attention as A then
 * B, in one append and one attend.
 *
 * Inputs (host arrays): L lanes; indptr_a/indptr_b [L+1]; slots_a [NA],
 * slots_b [NB]; kv_len_a/kv_len_b/fold_a/fold_b [L]; committed [L];
 * page_indptr_host [L+1]; page_size.
 * Outputs (host arrays, written only when eligible): indptr_m [L+1];
 * src_row [NA+NB]: merged row i is row src_row[i] of A if < NA, else row
 * src_row[i] - NA of B; row_of_a [NA], row_of_b [NB]: merged row of each
 * input row (for readout lists); kv_len_m, fold_m [L]. Positions, slots and
 * K/V/Q rows of M are A's and B's gathered by src_row.
 * Returns FP_OK when eligible, 1 when not (outputs untouched), FP_ERR_NULL /
 * FP_ERR_SHAPE for bad arguments.
 */
int fp_vertical_merge(int32_t L, const int32_t *indptr_a, const int32_t *slots_a, const int32_t *kv_len_a,
                      const int32_t *fold_a, const int32_t *indptr_b, const int32_t *slots_b,
                      const int32_t *kv_len_b, const int32_t *fold_b, const int32_t *committed,
                      const int32_t *page_indptr_host, int32_t page_size, int32_t *indptr_m, int32_t *src_row,
                      int32_t *row_of_a, int32_t *row_of_b, int32_t *kv_len_m, int32_t *fold_m);

/* ---- host-only accounting (Pie reviews, Eq. (1) and Eq. (2)) ---- */
uint64_t fp_kv_bytes(int32_t L, int32_t H_kv, int32_t d, uint64_t T, int32_t b); /* 2*L*H_kv*d*T*b   */
uint64_t fp_pages_for(uint64_t T, int32_t P);                                   /* ceil(T/P)        */
uint64_t fp_page_waste(uint64_t T, int32_t P);                                  /* P*ceil(T/P) - T  */
uint64_t fp_page_bytes(int32_t P, int32_t H_kv, int32_t d);                     /* 2*H_kv*P*d*2     */

/* Library version string (static storage). */
const char *fp_version(void);

/* SHA-256 (hex) of the library's source files as they were compiled (static
 * storage): a binding compares it with its sources to refuse a stale build. */
const char *fp_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* FP_H_ */
