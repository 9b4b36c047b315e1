/*
 * libtopktopp — per-row top-k / top-p logits filter for AMD Instinct MI355X (gfx950).
 *
 * What is computed. For every row b of a [B, V] logits matrix the filter
 * follows the eight steps of the CANN ops-nn page "ApplyTopKTopPWithSorted 的
 * top-k/top-p 采样过滤原理与 aclnn 调用指南" (cited below as AKP), §2:
 *   1-3. the k-th largest value of the row is the top-k threshold and every
 *        value strictly below it is masked;
 *   4-5. a softmax (fp32 or wider) of the surviving values is accumulated
 *        from the smallest probability upwards;
 *   6-7. every position whose cumulative probability is <= 1 - p[b] is masked,
 *        except the last (largest) position, which always survives;
 *   8.   the result is returned in the original vocabulary order.
 * The order is the stable ascending sort of the row: equal values (and -0.0
 * next to +0.0, which compare equal) keep their original index order, so at
 * a top-p boundary inside a run of equal values the lower indices are masked
 * first. A kept position holds the input bits unchanged; a masked position
 * holds the dtype's -inf (fp32 0xFF800000, fp16 0xFC00, bf16 0xFF80; AKP §6.3).
 *
 * Modes (AKP §4, §5.2). p and k are each optional, but not both. k[b] <= 0 or
 * k[b] >= V disables top-k for that row. p[b] >= 1 disables top-p in effect
 * (nothing with positive probability is masked); p[b] <= 0 keeps only the
 * last sorted position. Values of p are applied as given, without clamping.
 *
 * Numerics. t = 1 - p[b] is formed in fp32 from p widened exactly. The
 * cumulative probabilities are computed on the device in fp32/fixed-point
 * arithmetic whose summation order differs from a sequential sum; only
 * positions whose exact cumulative probability lies within about 1e-5 of t
 * can be decided differently from an exact evaluation. The top-k mask and
 * the kept values are exact. Results are deterministic: the same inputs give
 * the same output bits on every call.
 *
 * Memory and streams. Every data pointer is a device pointer owned by the
 * caller; nothing is retained after the call returns. Work is enqueued on
 * `stream` (a hipStream_t; NULL means the default stream) and the call
 * returns without synchronising. The library allocates no device memory
 * and the entry points never call hipMalloc. `out` must not overlap any input.
 * Rows are dense and row-major: element (b, v) sits at offset b * V + v,
 * except where an entry point takes strides (the _ex and _strided ones).
 *
 * Errors. Arguments are checked on the host before anything is enqueued, in
 * the order of the aclnn checks (AKP §5.3): null pointers first, then dtype,
 * then shape. On an error nothing is enqueued, and topktopp_last_error()
 * describes the problem. Device data (the values of p, k, sortedness) is not
 * validated.
 */
#ifndef TOPKTOPP_H
#define TOPKTOPP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits, sorted values, p and out (AKP §3 and §5.2 tables). */
typedef enum {
  TOPKTOPP_F32 = 0,
  TOPKTOPP_F16 = 1,
  TOPKTOPP_BF16 = 2
} topktopp_dtype;

/* Return codes, mirroring the aclnn ones of AKP §5.3. */
typedef enum {
  TOPKTOPP_OK = 0,
  TOPKTOPP_ERR_NULLPTR = 1, /* logits/sorted input/out is NULL, or p and k are both NULL (aclnn 161001) */
  TOPKTOPP_ERR_INVALID = 2, /* unsupported dtype, negative or too large shape, overlapping out (aclnn 161002) */
  TOPKTOPP_ERR_RUNTIME = 3  /* a HIP launch failed; the message names the HIP error */
} topktopp_status;

/* Largest supported row length, 2^20 (the same bound the companion sampling
 * operator, aclnnTopKTopPSampleV2, states for its vocabulary size). */
#define TOPKTOPP_MAX_V (1 << 20)

/* Largest supported number of rows, 2^31 - 1. Batches of more than 2^21
 * rows are launched in row chunks. */
#define TOPKTOPP_MAX_B 0x7FFFFFFFLL

/* Largest row stride accepted by the _ex entry points, in elements (2^31). */
#define TOPKTOPP_MAX_LD (1LL << 31)

/*
 * apply_top_k_top_p — filter raw logits (the aclnn entry of AKP §5 and §6.1,
 * which sorts internally). No sort is materialised: the threshold pair that
 * the stable sort would produce is found by radix selection.
 *
 *   logits  [B, V] device buffer of `dtype` values.
 *   dtype   one of topktopp_dtype.
 *   B, V    rows and row length; B == 0 or V == 0 is a successful no-op
 *           (every pointer may then be NULL; only dtype is checked);
 *           V == 1 copies logits to out (AKP §6.1); V <= TOPKTOPP_MAX_V,
 *           B <= TOPKTOPP_MAX_B.
 *   p       [B] device buffer of `dtype` values, or NULL for no top-p.
 *   k       [B] device buffer of int32, or NULL for no top-k.
 *   out     [B, V] device buffer of `dtype`, written completely.
 *   stream  hipStream_t to enqueue on, or NULL.
 */
topktopp_status apply_top_k_top_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V,
                                  const void* p, const int32_t* k, void* out, void* stream);

/*
 * apply_top_k_top_p_with_sorted — the sorted-input operator
 * ApplyTopKTopPWithSorted (AKP §1 and the §3 parameter table).
 *
 *   sorted_value    [B, V] device buffer, each row ascending.
 *   sorted_indices  [B, V] int32 device buffer, each row the permutation that
 *                   produced sorted_value from the original row. Positions in
 *                   this order decide ties.
 *   dtype, B, V, p, k, out, stream   as for apply_top_k_top_p.
 *   logits          [B, V] original (unsorted) values, or NULL. When given,
 *                   kept outputs are read from it in the original order and
 *                   sorted_value[b][j] must equal logits[b][sorted_indices[b][j]].
 *                   When NULL, out is written by scattering through
 *                   sorted_indices.
 * Sortedness and the permutation are the caller's contract and are not checked.
 */
topktopp_status apply_top_k_top_p_with_sorted(const void* sorted_value, const int32_t* sorted_indices,
                                              topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                              const int32_t* k, const void* logits, void* out,
                                              void* stream);

/*
 * apply_top_k_top_p_min_p — apply_top_k_top_p followed by the min-p stage of
 * Ascend's "aclnnTopKTopPSampleV2" page ("minP sampling"; cited as TKS).
 *
 *   min_p   [B] device buffer of `dtype` values (like p), or NULL for no
 *           min-p. Other arguments as for apply_top_k_top_p; p, k and min_p
 *           may each be NULL, but not all three (ERR_NULLPTR).
 *
 * Min-p takes the probabilities left after top-k and top-p (the softmax of
 * the top-k survivors, step 4 above) and masks every position whose
 * probability is strictly below the largest one times min_p[b]; as the
 * ratio of two of those probabilities is exp(x - x_max), a position survives
 * iff exp(x - x_max) >= min_p[b]. min_p[b] <= 0 (or NaN) skips the stage;
 * min_p[b] >= 1 keeps a single position, the maximum with the highest
 * original index (TKS keeps one token with the maximum value; this takes the
 * stable order's last one, as p <= 0 does). Each stage masks a prefix of the
 * stable ascending order, so the survivors are those of all stages at once.
 *
 * Numerics. exp is taken in fp32 on the device; only positions whose exact
 * ratio lies within a relative 1e-5 of min_p[b] can be decided differently
 * from an exact evaluation.
 */
topktopp_status apply_top_k_top_p_min_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V,
                                        const void* p, const int32_t* k, const void* min_p, void* out,
                                        void* stream);

/*
 * apply_top_k_top_p_min_p_with_sorted — apply_top_k_top_p_with_sorted
 * followed by the min-p stage described for apply_top_k_top_p_min_p.
 *   min_p   [B] device buffer of `dtype` values, or NULL. Other arguments as
 *           for apply_top_k_top_p_with_sorted; p, k and min_p may each be
 *           NULL, but not all three.
 */
topktopp_status apply_top_k_top_p_min_p_with_sorted(const void* sorted_value, const int32_t* sorted_indices,
                                                    topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                                    const int32_t* k, const void* min_p, const void* logits,
                                                    void* out, void* stream);

/*
 * apply_top_k_top_p_ex — apply_top_k_top_p_min_p on row-strided operands: row
 * b of logits starts at element b * ld_logits and row b of out at element
 * b * ld_out (a [B, V] view of a wider buffer, e.g. a vocabulary padded to a
 * multiple of 64; the aclnn entry makes such views contiguous first, AKP
 * §6.1). Elements within a row are contiguous. Each stride must be >= V and
 * <= TOPKTOPP_MAX_LD (else ERR_INVALID); the strided extents of out and the
 * inputs must not overlap. Positions between V and the stride are neither
 * read nor written. Other arguments as for apply_top_k_top_p_min_p.
 */
topktopp_status apply_top_k_top_p_ex(const void* logits, int64_t ld_logits, topktopp_dtype dtype, int64_t B, int64_t V,
                                     const void* p, const int32_t* k, const void* min_p, void* out,
                                     int64_t ld_out, void* stream);

/*
 * apply_top_k_top_p_strided — apply_top_k_top_p_min_p on arbitrary strided
 * views (the aclnn entry accepts non-contiguous tensors and makes them
 * contiguous before filtering, AKP §6.1; this reads and writes the views in
 * place instead). All strides are in elements:
 *   logits  element (b, v) at logits[b * logits_row_stride + v * logits_col_stride];
 *   out     element (b, v) at out[b * out_row_stride + v * out_col_stride];
 *   p, k, min_p   entry b at p[b * p_stride], k[b * k_stride],
 *           min_p[b * min_p_stride] (a stride of 0 shares one value among
 *           all rows; the stride of a NULL operand is ignored).
 * E.g. a [V, B] buffer filtered as its transpose passes row stride 1 and
 * column stride B. Input strides must lie in [0, TOPKTOPP_MAX_LD]; out's in
 * [1, TOPKTOPP_MAX_LD] (ignored along an extent of 1), and out must give
 * every (b, v) its own element: one of its strides must be at least the
 * other times that other dimension's extent (out_row_stride >= V *
 * out_col_stride, or out_col_stride >= B * out_row_stride), else
 * ERR_INVALID. The byte span of out (from its first to its last element)
 * must not overlap the span of any input. Elements of the spans that belong
 * to no (b, v) are neither read nor written. Other arguments, checks and
 * results as for apply_top_k_top_p_min_p (p, k and min_p may each be NULL,
 * but not all three).
 *
 * When rows are contiguous (logits_col_stride == out_col_stride == 1, row
 * strides >= V) and p, k and min_p are dense, this is apply_top_k_top_p_ex.
 * Otherwise every element is accessed on its own by a streamed kernel, which
 * is several times slower than the vector path of contiguous rows.
 */
topktopp_status apply_top_k_top_p_strided(const void* logits, int64_t logits_row_stride, int64_t logits_col_stride,
                                          topktopp_dtype dtype, int64_t B, int64_t V, const void* p, int64_t p_stride,
                                          const int32_t* k, int64_t k_stride, const void* min_p,
                                          int64_t min_p_stride, void* out, int64_t out_row_stride,
                                          int64_t out_col_stride, void* stream);

/*
 * apply_top_k_top_p_with_sorted_ex — apply_top_k_top_p_min_p_with_sorted on
 * row-strided operands, one row stride (in elements) per [B, V] operand, with
 * the rules of apply_top_k_top_p_ex. ld_logits is ignored when logits is NULL.
 */
topktopp_status apply_top_k_top_p_with_sorted_ex(const void* sorted_value, int64_t ld_sorted_value,
                                                 const int32_t* sorted_indices, int64_t ld_sorted_indices,
                                                 topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                                 const int32_t* k, const void* min_p, const void* logits,
                                                 int64_t ld_logits, void* out, int64_t ld_out, void* stream);

/*
 * sample_top_k_top_p — the filter (top-k, top-p, min-p as in
 * apply_top_k_top_p_min_p) followed by the sampling stage of TKS
 * ("Subsequent processing"), one index per row. probs are the filtered
 * probabilities in descending order; descending order is the reverse of the
 * stable ascending order, so among equal values the higher original index
 * comes first.
 *
 *   logits, dtype, B, V, p, k, min_p   as for apply_top_k_top_p_min_p, except
 *            that p, k and min_p may all be NULL (sampling from the whole row).
 *   q        [B, V] fp32 device buffer, or NULL.
 *            NULL ("None" mode): selected[b] is the index of the first
 *            maximum of probs, the maximum value with the highest index.
 *            Given ("QSample"): selected[b] is the index of the first maximum
 *            of probs / (q[b][r] + eps), q[b][r] pairing with the survivor of
 *            descending rank r; only the first n_b entries of a row are read,
 *            n_b being the row's survivor count.
 *   eps      added to q; finite and >= 0 (the pages give it no value).
 *   out      [B, V] device buffer for the filtered logits, or NULL to skip
 *            them (then the row is only read, not written).
 *   selected [B] int32 device buffer, written completely, with an index in
 *            [0, V) for every row, whatever its number of survivors.
 * Errors as for apply_top_k_top_p_min_p; selected NULL is ERR_NULLPTR, a
 * negative or non-finite eps ERR_INVALID, and out or selected overlapping
 * another buffer ERR_INVALID.
 */
topktopp_status sample_top_k_top_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                   const int32_t* k, const void* min_p, const float* q, float eps, void* out,
                                   int32_t* selected, void* stream);

/*
 * top_k_top_p_sorted_survivors — the filter (as apply_top_k_top_p_min_p)
 * returning the survivors themselves, in descending order, instead of the
 * filtered row: the intermediate output of TKS (logitsSortMasked and
 * logitsIdx, "Intermediate result output"), cut to the survivors. For row b
 * and descending rank r < min(n_b, cap), with n_b the row's survivor count:
 *   probs[b][r]    the survivor's probability of step 4 (the softmax over the
 *                  top-k survivors, fp32), or skipped when probs is NULL;
 *   indices[b][r]  its original index (int32);
 * ranks n_b .. cap-1 hold probability 0 and index -1; counts[b] = n_b (which
 * may exceed cap). Descending order is the reverse of the stable ascending
 * order (equal values: higher index first). p, k and min_p may each be NULL.
 *   cap     entries per output row, 1 <= cap <= 2^20 (else ERR_INVALID).
 *   probs   [B, cap] fp32 device buffer, or NULL.
 *   indices [B, cap] int32 device buffer.
 *   counts  [B] int32 device buffer.
 * Every row lists min(n_b, cap) survivors, whatever n_b is (up to V).
 * Errors as for apply_top_k_top_p_min_p; outputs may not overlap inputs or
 * each other (ERR_INVALID).
 */
topktopp_status top_k_top_p_sorted_survivors(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                             const int32_t* k, const void* min_p, int64_t cap, float* probs,
                                             int32_t* indices, int32_t* counts, void* stream);

/* Text of the most recent error on the calling thread ("" if none); the
 * counterpart of aclGetRecentErrMsg (AKP §8). Valid until the next call on
 * the same thread. */
const char* topktopp_last_error(void);

/*
 * Launch-plan override, for tests and measurement. policy 0 (default) lets
 * the library choose: the candidate plan, with the row held in registers
 * when it fits; 1 forces the multi-pass plan for every row; 2 forces the
 * candidate plan with the row re-read from global memory. Every policy
 * computes the same filter; top-p decisions may differ only inside the
 * tolerance band described above. Returns the previous policy, or -1 for an
 * unknown value (which is ignored). The setting is process-wide.
 */
int topktopp_set_plan_policy(int policy);

#ifdef __cplusplus
}
#endif

#endif /* TOPKTOPP_H */
