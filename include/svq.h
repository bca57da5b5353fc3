/*
 * libsvq - spherical vector quantization (SVQ) decode-and-multiply for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one described in "SAGE: Pushing 2-Bit Vector-Quantized
 * LLMs toward Real-World Usability" (cited below as "SAGE").  Each subvector
 * of 8 weights is coded as 8 sign bits, a direction index into a per-matrix
 * codebook and an index into a per-matrix table of quantized radii, with a
 * per-matrix split of 10 index bits between the two (SAGE, Fig. 2 caption;
 * 18 bits per 8 weights = 2.25 bits per weight, SAGE Table 1, SPHQuant row).
 * Weights are rebuilt on demand inside the product, never stored decoded
 * (SAGE, Fig. 1 and Fig. 5 captions), and the 8 inputs of a subvector are
 * reordered activations (SAGE, Fig. 6 caption).
 *
 * Canonical input format (the pages leave it open; this is the library's
 * contract, identical to the CPU oracle shipped with the tests):
 *
 *   - code g = i*(k/8) + c covers row i, permuted slots 8c..8c+7, and occupies
 *     bits [18g, 18g+18) of the code stream; stream bit t is bit (t % 8) of
 *     byte t / 8 (LSB first, rows back to back, no padding);
 *   - inside a code, LSB first: bits 0-7 signs (bit l for lane l, 1 means
 *     negative), then bd direction bits, then br = 10 - bd radius bits;
 *   - decoded weight: What[i, perm[8c+l]] = R[r] * (-1)^{s_l} * D[d][l],
 *     where D is the (1<<bd) x 8 fp16 direction codebook and R the (1<<br)
 *     fp16 radius table; slot p of the permuted order takes input channel
 *     perm[p] (a gather permutation);
 *   - y[m, i] = sum_j What[i, j] * x[m, j]  with x bf16, y bf16 or fp32.
 *
 * Numerics.  For m <= 16 (the batch-1 and small-batch paths) each decoded
 * weight is the exact fp32 product R*D (fp16 x fp16 fits in 22 bits) and
 * accumulation is fp32: for m <= 4 the radius multiplies an fp16 dot
 * product in fp32; for 4 < m <= 16 the weight enters the matrix cores as
 * two fp16 halves whose sum is R*D*2^s exactly (s per matrix, chosen and
 * verified by svq_pack; tables that admit no such split are multiplied
 * four activation rows at a time by the m <= 4 kernels instead).  The activations enter the dot products as fp16
 * after a power-of-two scale chosen per 512-slot block of permuted inputs
 * (per row of x): the block's largest magnitude is scaled into [2^14, 2^15),
 * which keeps every bf16 value of magnitude at least 2^-31 times that
 * largest one exact; smaller values round to fp16 subnormals (an absolute
 * error of at most 2^-39 times the block's largest magnitude).  For m > 16
 * (the dequant GEMM on the matrix cores) a weight enters as RNE_bf16(R*D)
 * with its sign, x as bf16, accumulation fp32.  bf16 outputs are rounded to
 * nearest even.
 *
 * Ownership.  The caller owns every byte: the packed matrix buffer and the
 * workspace are device memory the caller allocates (size queries below);
 * handles are plain structs held by the caller.  The library allocates no
 * device memory and keeps no state, with one exception: the fixed scratch
 * array of svq_linear_noalloc (SVQ_SCRATCH_BYTES per device, held until the
 * process ends).  There is nothing to free.
 *
 * Errors.  Every call returns an svq_status and never aborts.  Arguments are
 * validated before any device work.  HIP errors map to SVQ_ERR_HIP.  All
 * device work is asynchronous on the given stream (NULL = default stream),
 * except that svq_pack waits for its own copies before returning.
 *
 * Streams: `stream` arguments are hipStream_t values passed as void*.
 */
#ifndef SVQ_H
#define SVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVQ_OK = 0,
  SVQ_ERR_INVALID_ARG = -1,      /* null pointer, bad size, not a permutation ... */
  SVQ_ERR_UNSUPPORTED = -2,      /* bd outside {6,7,8}, shape beyond the limits */
  SVQ_ERR_BUFFER_TOO_SMALL = -3, /* dst / workspace smaller than required       */
  SVQ_ERR_HIP = -4               /* a HIP runtime call or launch failed          */
} svq_status;

typedef enum { SVQ_BF16 = 0, SVQ_F32 = 1 } svq_dtype;

/* Limits checked by svq_pack. */
#define SVQ_MAX_K 65536 /* the permutation is stored as uint16 */
#define SVQ_MAX_N (1 << 24)

/* One SVQ-coded matrix in canonical form.  HOST pointers, read only.
 * n: output rows; k: input channels, k % 8 == 0; bd + br == 10, bd in {6,7,8}
 * (direction codebook <= 4 KB; SAGE Fig. 2 caption: the split is chosen per
 * matrix).  codes: n*(k/8) 18-bit fields as described above, ceil(n*k*9/32)
 * bytes.  dir_codebook: (1<<bd) rows of 8 fp16 bit patterns, row-major.
 * radius_table: (1<<br) fp16 bit patterns.  perm: k distinct values in
 * [0, k). */
typedef struct {
  int32_t n, k;
  int32_t bd, br;
  const uint8_t *codes;
  const uint16_t *dir_codebook;
  const uint16_t *radius_table;
  const int32_t *perm;
} svq_matrix_desc;

/* A packed matrix: a caller-owned POD that names a caller-owned device
 * buffer.  Filled by svq_pack; read by svq_linear / svq_moe_linear.  The
 * offsets are byte offsets from `dev`. */
typedef struct {
  void *dev;
  int32_t n, k, bd, br;
  int32_t n_tiles;   /* ceil(n / 16) row tiles                         */
  int32_t units;     /* code units per row tile: ceil(k / 512)          */
  uint64_t off_dtab; /* 256 x 8 fp16: direction rows by low index byte  */
  uint64_t off_rtab; /* 16 fp16: radius by radius index (zero padded)   */
  uint64_t off_btab; /* 1024 x 8 bf16: RNE_bf16(R[r] * D[d][l]) by index */
  uint64_t off_xtab; /* 1024 x (8 + 8) fp16: hi + lo = R[r]*D[d][l]*2^xscale_log2 exactly */
  uint64_t off_perm; /* k uint16 slots -> channels                      */
  uint64_t off_codes;/* n_tiles * units * 2304 bytes of coded units     */
  uint64_t code_bytes;    /* canonical code bytes: ceil(n*k*9/32)       */
  uint64_t padded_code_bytes; /* bytes of coded units including padding  */
  uint64_t bytes;    /* total packed buffer size                         */
  int32_t xscale_log2; /* the power of two of the exact split, or
                          SVQ_NO_EXACT_SPLIT when the tables admit none    */
  int32_t reserved;
} svq_handle;
#define SVQ_NO_EXACT_SPLIT (-2147483647 - 1)

/* svq_pack: one-time repack of a canonical matrix into the kernel layout
 * (SAGE Fig. 2 caption for what a code holds; the layout itself keeps the
 * 18 bits per 8 weights and only regroups them for 128-bit loads).
 *   src:        canonical matrix (host memory).
 *   dst_dev:    device buffer of at least *dst_bytes bytes, or NULL to only
 *               query the size.
 *   dst_bytes:  in: capacity of dst_dev (ignored when dst_dev is NULL);
 *               out: bytes required.
 *   out:        filled on success when dst_dev is not NULL (may be NULL for a
 *               size query).
 * Validates src fully (including that perm is a permutation) before any
 * device work.  Copies on `stream` and synchronizes it before returning, so
 * the host arrays may be freed afterwards. */
svq_status svq_pack(const svq_matrix_desc *src, void *dst_dev, size_t *dst_bytes,
                    svq_handle *out, void *stream);

/* svq_linear: y = x * What^T for one packed matrix (SAGE Fig. 1 / Fig. 5
 * captions: weights reconstructed on demand; Fig. 6 caption: reordered
 * activations gathered per subvector).  Beside the operands the call takes a
 * workspace pair: the library never allocates device memory, so the scratch
 * some shapes need (permuted activations, K-split partial sums) comes from
 * the caller, sized by a query call with workspace == NULL.
 *   w:          packed matrix.
 *   x:          device bf16 [m][ldx], ldx >= k.
 *   m:          rows of x, >= 1.
 *   y:          device [m][ldy] of type ydt, ldy >= n.
 *   workspace:  device scratch of at least *workspace_bytes bytes, or NULL to
 *               query the size (then nothing is launched).
 * The workspace holds the permuted activations of this call; calls that
 * share a workspace must be ordered on one stream.  x, y and the workspace
 * must not overlap. */
svq_status svq_linear(const svq_handle *w, const void *x, int64_t m, int64_t ldx,
                      void *y, int64_t ldy, svq_dtype ydt,
                      void *workspace, size_t *workspace_bytes, void *stream);

/* svq_linear_batched: svq_linear for `count` (1..8) independent matrices
 * that share m, e.g. the linears of one decoder layer, in one call (a single
 * kernel launch when m <= 4).  Arrays are host arrays of length count:
 * w[j] (packed matrices, shapes may differ), x[j] / ldx[j] (device bf16
 * inputs), y[j] / ldy[j] (device outputs of type ydt).  The workspace query
 * (workspace == NULL) only needs w, count, m and ydt; ldx / ldy are checked
 * when given.  Same numerics, ownership and error rules as svq_linear. */
svq_status svq_linear_batched(const svq_handle *w, int32_t count, const void *const *x,
                              const int64_t *ldx, int64_t m, void *const *y, const int64_t *ldy,
                              svq_dtype ydt, void *workspace, size_t *workspace_bytes,
                              void *stream);

/* svq_linear_noalloc: svq_linear without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid hipMalloc).  The scratch svq_linear would take
 * from the caller comes from a file-scope device array of SVQ_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends; the
 * call itself allocates nothing (no hipMalloc, no allocating library call).
 *   w, x, m, ldx, y, ldy, ydt, stream:  as for svq_linear.
 * Returns SVQ_ERR_UNSUPPORTED, before any device work, when the call would
 * need more scratch than SVQ_SCRATCH_BYTES (svq_linear's workspace query
 * gives the size).  Every call on one GPU shares that GPU's array and it
 * keeps the last call's contents: calls that overlap on one GPU (different
 * streams, different host threads without ordering) race and give undefined
 * results.  Results equal svq_linear's for the same arguments. */
#define SVQ_SCRATCH_BYTES ((size_t)64 << 20)
svq_status svq_linear_noalloc(const svq_handle *w, const void *x, int64_t m, int64_t ldx,
                              void *y, int64_t ldy, svq_dtype ydt, void *stream);

/* svq_moe_linear: one projection of a routed mixture of experts, one output
 * row per routed (token, expert) slot; the grouped form of svq_linear.  The
 * pages code dense linears only; this call applies the same per-matrix
 * format to each expert's matrices (each expert with its own codebook,
 * radius table, permutation and split) under the usual top-k slot
 * convention below, which is this library's definition, not the pages'.
 *   experts:      host array of num_experts packed matrices, all with the
 *                 same n and k (bd may differ per expert).
 *   x:            device bf16; row t (token) when x_per_slot == 0, row
 *                 q = t*topk + j (slot) when x_per_slot == 1; stride ldx.
 *   expert_ids:   device int32 [m*topk]; slot q = t*topk + j uses expert
 *                 expert_ids[q], each in [0, num_experts).  A slot whose id
 *                 is outside that range is skipped: its output row is
 *                 written as zeros and no memory outside the arguments is
 *                 touched.
 *   y:            device [m*topk][ldy] of type ydt, slot-major.
 *   workspace:    as for svq_linear (routing tables and permuted inputs).
 * Numerics: up to 64 slots (m*topk <= 64) every slot runs the exact batch-1
 * product of its expert (the m <= 4 numerics above); beyond that the slots
 * are grouped by expert (work items of at most 48 rows) and each weight
 * enters the matrix cores as RNE_bf16(R*D) with its sign, x as bf16,
 * accumulation fp32 (the m > 16 numerics).
 * Routing weights, the activation between projections and the combine over
 * a token's experts are the caller's. */
svq_status svq_moe_linear(const svq_handle *experts, int32_t num_experts,
                          const void *x, int64_t ldx, int32_t x_per_slot,
                          const int32_t *expert_ids, int64_t m, int32_t topk,
                          void *y, int64_t ldy, svq_dtype ydt,
                          void *workspace, size_t *workspace_bytes, void *stream);

/* svq_moe_linear_batched: svq_moe_linear for `count` (1..4) projections that
 * share the routing (expert_ids, m, topk, x_per_slot), e.g. the gate and up
 * projections of one FFN, which read the same token rows.  Up to 64 slots
 * one kernel launch serves every projection; up to 8192 slots one
 * activation-staging launch and one product launch serve every projection
 * (the routing is worked out once); beyond that the projections run one
 * after another.
 *   experts:      host array of count pointers; experts[c] is a host array
 *                 of num_experts packed matrices of projection c (one n and k
 *                 per projection; projections may differ).
 *   num_experts:  1..256, and count * num_experts <= 256
 *                 (SVQ_ERR_UNSUPPORTED otherwise).
 *   x, ldx:       host arrays of count device bf16 inputs and their strides
 *                 (rows as in svq_moe_linear; the same pointer may repeat).
 *   y, ldy:       host arrays of count device outputs of type ydt,
 *                 [m*topk][ldy[c]] each, slot-major.
 *   workspace:    as for svq_moe_linear; the query (workspace == NULL)
 *                 needs only experts, count, num_experts, m, topk,
 *                 x_per_slot and ydt (x, ldx, y, ldy may then be NULL).  Up
 *                 to 8192 slots it holds the routing once and the staged
 *                 activations of every projection; beyond, it is the
 *                 largest any single projection needs, used in turn.
 * The outputs must not overlap one another, the inputs or the workspace
 * (inputs may be shared).  Results, numerics, the treatment of ids outside
 * [0, num_experts) and the error rules are those of count separate
 * svq_moe_linear calls with the same arguments, in order, on the same
 * stream. */
svq_status svq_moe_linear_batched(const svq_handle *const *experts, int32_t count,
                                  int32_t num_experts, const void *const *x,
                                  const int64_t *ldx, int32_t x_per_slot,
                                  const int32_t *expert_ids, int64_t m, int32_t topk,
                                  void *const *y, const int64_t *ldy, svq_dtype ydt,
                                  void *workspace, size_t *workspace_bytes, void *stream);

/* svq_encode: the codes of a float weight matrix for given tables -- the
 * step before svq_pack (SAGE Fig. 2 caption: each 8-weight subvector, taken
 * along the channel permutation, is coded by its signs, a direction index
 * into the codebook and a quantized radius).  Subvector c of row i is
 * v[l] = w[i][perm[8c + l]] and its code (bits 0-7 signs, then bd direction
 * bits, then 10 - bd radius bits, as in svq_matrix_desc) is:
 *   sign bit l  = the IEEE sign bit of v[l] (1 for negatives and -0.0);
 *   direction   = the codebook row j with the largest
 *                 sum_l |v[l]| * D[j][l], the first such row on ties;
 *   radius      = the table entry nearest to the norm of v, the lower entry
 *                 on ties.
 * Scores and squared norms are formed in double precision, lane order
 * 0..7, without fused multiply-adds; the radius is decided by the squared
 * norm against the squared midpoints of consecutive radii.
 *   w:          device fp32 [n][ldw], ldw >= k; every value finite.
 *   n, k:       k a multiple of 8, limits as for svq_pack.
 *   bd:         direction-index bits, 6..8 (radius bits 10 - bd).
 *   codebook:   host, (1 << bd) x 8 fp16 bit patterns, finite.
 *   radius:     host, 1 << (10 - bd) fp16 bit patterns, finite, >= 0 and
 *               strictly increasing.
 *   perm:       host, k entries, a permutation of [0, k).
 *   codes:      device, out: the canonical LSB-first stream of the n*k/8
 *               codes, ceil(n*k*9/32) bytes (the svq_matrix_desc format).
 *   workspace:  device scratch of at least *workspace_bytes bytes (the
 *               tables are staged there), or NULL to query the size.
 * Validates every host argument before any device work; copies the tables
 * on `stream` and synchronizes it before returning (the host arrays may be
 * freed afterwards).  Non-finite weights make the codes undefined. */
svq_status svq_encode(const float *w, int64_t ldw, int32_t n, int32_t k, int32_t bd,
                      const uint16_t *codebook, const uint16_t *radius, const int32_t *perm,
                      void *codes, void *workspace, size_t *workspace_bytes, void *stream);

/* svq_encode_weighted: as svq_encode, but each code is chosen by
 * activation-weighted fitting (SAGE abstract and Fig. 2 caption: ESG
 * protects sensitive channels through fitting weighted by calibration
 * activations).  The pages give no formula; this library's reading: with
 * h_l = h[perm[8c + l]] the weight of the input channel at lane l, the code
 * minimises sum_l h_l (v[l] - w_hat[l])^2 over every (direction, radius)
 * pair.  Signs are those of svq_encode (a decoded weight with the sign of
 * v[l] is never farther from it).  With a_l = |v[l]|, the pair (d, r)
 * minimising the code-dependent part
 *   E = (R[r] * R[r]) * B_d - (R[r] + R[r]) * A_d,
 *   A_d = sum_l (h_l * a_l) * D[d][l],  B_d = sum_l (h_l * D[d][l]) * D[d][l]
 * is chosen, pairs in order (d ascending, then r ascending), the first
 * minimum on ties; double precision, lanes added in order 0..7, no fused
 * multiply-adds.
 *   w, ldw, n, k, bd, codebook, radius, perm, codes, workspace, stream:
 *               as for svq_encode (the radius table is checked the same way).
 *   h:          device double [k]: the weight of input channel j (e.g. the
 *               ESG energy raised to an exponent), finite and >= 0 (other
 *               values make the codes undefined); NULL only in a size query.
 * Validates every host argument before any device work and synchronizes
 * `stream` before returning. */
svq_status svq_encode_weighted(const float *w, int64_t ldw, int32_t n, int32_t k, int32_t bd,
                               const uint16_t *codebook, const uint16_t *radius,
                               const int32_t *perm, const double *h, void *codes,
                               void *workspace, size_t *workspace_bytes, void *stream);

/* svq_esg_perm: Energy-Stratified Grouping -- the channel permutation of a
 * matrix from calibration activations of its input (SAGE abstract and
 * Fig. 2 caption: channel energies from calibration activations; every
 * subvector takes channels from different energy tiers).  Readings:
 *   energy[j] = (x[0][j]^2 + x[1][j]^2 + ... + x[t-1][j]^2) / t, in double
 *               precision, token order, one division at the end;
 *   ranks:      channels by decreasing energy, equal energies by increasing
 *               index; tier l = ranks [l*k/8, (l+1)*k/8);
 *   perm:       slot 8c + l <- the channel of rank l*(k/8) + c, so lane l
 *               of every subvector comes from tier l (the svq_matrix_desc
 *               gather convention: slot p reads channel perm[p]).
 *   x:          device bf16 [t][ldx], t >= 1; x and ldx*2 16-byte aligned
 *               (ldx a multiple of 8, ldx >= k); every value finite.
 *   k:          a multiple of 8, at most the svq_pack limit.
 *   energy:     device double [k], out.
 *   perm:       device int32 [k], out.
 *   workspace:  device scratch of at least *workspace_bytes bytes (4k), or
 *               NULL to query the size.
 * Asynchronous on `stream`.  Non-finite activations make the outputs
 * undefined (perm stays a map into [0, k)). */
svq_status svq_esg_perm(const void *x, int64_t t, int64_t ldx, int32_t k, double *energy,
                        int32_t *perm, void *workspace, size_t *workspace_bytes, void *stream);

/* svq_abs_select: Adaptive Bit Split -- encode one matrix under each
 * candidate split and keep the one with the lowest activation-weighted
 * reconstruction error (SAGE abstract and Fig. 2 caption).  Every candidate
 * is coded by the svq_encode rule, or by the svq_encode_weighted rule with
 * the same h when weighted_fit is 1; its error is
 *   sum over rows i (row order) of
 *     sum over subvectors c (code order) of
 *       sum over lanes l (lane order) of (v[l] - w_hat[l])^2 * h[perm[8c+l]]
 * with v[l] = w[i][perm[8c + l]] and w_hat the decoded weight, all in
 * double precision without fused multiply-adds.  The first candidate with
 * the smallest error wins.
 *   w, ldw, n, k, perm:  as for svq_encode (perm on the host).
 *   h:          device double [k]: the weight of input channel j (e.g. the
 *               ESG energy raised to an exponent), finite, >= 0.
 *   n_cand:     1..8 candidates: bd[c] (6..8), codebooks[c] and radii[c]
 *               (host tables as for svq_encode).
 *   weighted_fit: 0 (plain coding rule) or 1 (activation-weighted fit).
 *   codes:      device, out: the chosen candidate's code stream.
 *   chosen:     host, out: index of the chosen candidate.
 *   errors:     host, out: the error of every candidate [n_cand].
 *   workspace:  device scratch of at least *workspace_bytes bytes (tables,
 *               every candidate's codes and errors), or NULL to query.
 * Validates every host argument before any device work, then synchronizes
 * `stream` (the choice is made on the host from the device totals). */
svq_status svq_abs_select(const float *w, int64_t ldw, int32_t n, int32_t k, const double *h,
                          const int32_t *perm, int32_t n_cand, const int32_t *bd,
                          const uint16_t *const *codebooks, const uint16_t *const *radii,
                          int32_t weighted_fit, void *codes, int32_t *chosen, double *errors,
                          void *workspace, size_t *workspace_bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *svq_status_string(svq_status s);

#ifdef __cplusplus
}
#endif

#endif /* SVQ_H */
