/*
 * sag.h -- C ABI of the MI355X (gfx950) GNN-layer hot path.
 *
 * One GNN layer's work on one GPU's share of a graph: pull halo rows from a
 * stale-representation buffer, aggregate with a normalised sparse matrix
 * (CSR SpMM), transform with a dense matrix (MFMA GEMM, bias and ReLU fused),
 * and the backward pass (weight-gradient GEMM and the transposed SpMM).
 *
 * Sources (the four pages this library follows):
 *  - "Reducing Communication in Graph Neural Network Training" (CAGNET
 *    page), background section on GNN training: A gets self connections and
 *    is normalised as D^-1/2 (A+I) D^-1/2 with D the modified degrees; a
 *    layer computes sigma(A^T H W); SpMM and the dense product dominate and
 *    backpropagation uses the same primitives.  Its 1D block-row section: one
 *    process owns n/P consecutive rows.
 *  - Sylvie (1-bit quantised halo communication): "Graph Engine" builds the
 *    HALO node set of each partition; "Forward Propagation" multiplies the
 *    normalised adjacency with the concatenation of local and recovered halo
 *    rows; "Backward Propagation" sends the halo rows of the feature
 *    gradient back to their owners.
 *  - DIGEST (periodic stale representation synchronisation): the forward
 *    pass on a subgraph is P_in H_in + P_out H~_out with P_m = P_in + P_out;
 *    the "pull" operation copies H~_out from the stale store.
 *  - A DistDGL review: partitioning is done once and amortised over training.
 *
 * Conventions
 * -----------
 *  - Edge u -> v means node v aggregates u: CSR row v lists its sources u
 *    (the CAGNET page's A^T H).
 *  - Dense matrices are row-major with a leading dimension `ld` counted in
 *    elements.  Every dense pointer must be 16-byte aligned and ld times the
 *    element size a multiple of 16 bytes (SAG_E_ALIGN otherwise).  Padding
 *    elements (columns d .. ld-1) may hold anything: they are read only to
 *    fill 16-byte vectors and never enter a result, and they are never
 *    written.
 *  - bf16 data is passed as uint16_t bit patterns.  Every conversion from
 *    fp32 to bf16 rounds to nearest, ties to even.
 *  - Pointers are DEVICE pointers unless the comment says "host".  `stream`
 *    is a hipStream_t passed as void* (NULL = the null stream).
 *  - Ownership: the caller allocates every buffer, including the workspace
 *    `ws` whose size the matching *_workspace_bytes function returns (those
 *    functions run on the host only).  The library allocates no device
 *    memory and keeps no mutable state that a computation depends on: every
 *    choice (dtype, fusion, normalisation kind) is an argument of the call or
 *    a field of the caller's sag_csr, so it may be called from several host
 *    threads on different streams.  The opt-in measurement trace is per host
 *    thread and changes no result.  Launch settings (occupancy, CU count,
 *    LDS limits) are queried once per process, so the devices one process
 *    uses must be of one kind.
 *  - Errors: arguments are validated on the host before anything is
 *    launched; a failure returns a negative sag_status and launches nothing.
 *    A HIP error returns SAG_E_HIP.  sag_last_error() gives a detail string
 *    for the calling thread.  CSR contents (ordering, index ranges) are not
 *    re-validated by compute calls: a CSR that did not come from
 *    sag_csr_build_normalize (or equal one) gives undefined results.
 *  - Every call is asynchronous on `stream` except those documented as
 *    synchronising (sag_csr_build_normalize and its query, sag_csr_schedule
 *    and sag_csr_hub_split).
 *  - Results are deterministic: the same inputs, sizes and schedule give
 *    the same bits on every run (no floating-point atomics).
 */
#ifndef SAG_H
#define SAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SAG_OK = 0,
    SAG_E_INVALID = -1,      /* null pointer, bad size or range, bad enum     */
    SAG_E_ALIGN = -2,        /* pointer or leading dimension not 16-B aligned */
    SAG_E_WORKSPACE = -3,    /* workspace or output capacity too small        */
    SAG_E_RANGE = -4,        /* an edge id outside [0, n_global)              */
    SAG_E_HIP = -5,          /* a HIP runtime error                           */
    SAG_E_UNSUPPORTED = -6   /* a size or dtype combination not implemented  */
} sag_status;

typedef enum { SAG_F32 = 0, SAG_BF16 = 1 } sag_dtype;

/* Normalisation of the adjacency (the values stored in the CSR).
 * SAG_NORM_GCN : entry (r, c) = 1 / sqrt(d_r * d_c), d = degrees of A + I
 *                (CAGNET page, background; Sylvie, "Forward Propagation").
 * SAG_NORM_MEAN: entry (r, c) = 1 / d_r (GraphSAGE mean aggregator).
 * SAG_NORM_NONE: entry = 1.
 * Values are computed in fp64 with correctly rounded sqrt and divide and
 * rounded once to fp32; degrees below 1 are taken as 1. */
typedef enum { SAG_NORM_GCN = 0, SAG_NORM_MEAN = 1, SAG_NORM_NONE = 2 } sag_norm;

/* Build flags. */
enum {
    SAG_SYMMETRIZE = 1,   /* also use the reverse of every edge              */
    SAG_SELF_LOOPS = 2    /* add one self connection per local row (A + I)  */
};

/* A CSR matrix in device memory (host struct of device pointers), with an
 * optional degree-binned schedule.
 *
 * indptr[n_rows + 1] (int64), indices[nnz] (int32, column ids in
 * [0, n_cols), ascending within a row), values[nnz] (fp32; NULL = all 1).
 *
 * Schedule (sag_csr_schedule fills it; sched == NULL means none): the rows
 * are ordered by length class (floor(log2(len))), ascending row id within a
 * class, and split in three bins: short rows (len <= 32) are summed by a
 * group of lanes each, several rows per wavefront; medium rows (32 < len <=
 * seg_len) by one wavefront each; long rows (len > seg_len) are cut into
 * segments of seg_len entries, each summed by its own wavefront, and the
 * segment sums of a row are then added in segment order.  `sched` points to
 * 4 * n_rows int32 row records {row, len, start_lo, start_hi} in bin order,
 * then 4 * n_seg segment records {long row index, start_lo, start_hi, len},
 * then n_long + 1 int32 prefix counts of segments per long row.  Without a
 * schedule every row is treated as a medium row in natural order (correct,
 * slow on power-law degree laws).
 *
 * row_mean: nonzero says that every entry of row r holds 1/len(r) rounded
 * once to fp32 (the A that sag_csr_build_normalize writes with
 * SAG_NORM_MEAN; not its transpose).  Products over such a matrix read only
 * its pattern and scale each row's sum by that value, once per row instead
 * of once per entry; the result differs from reading the values only by
 * fp32 rounding.  Zero (also for any transpose): the stored values are
 * read.
 *
 * hub_part, cold_part (both or neither; host pointers): a hub split of this
 * matrix (sag_csr_hub_split): two CSRs over the same rows and columns, the
 * first holding the entries that fall in the columns with the most entries,
 * the second the rest, each row's entries in their order in this matrix and
 * with their values (row_mean 0, any schedule of their own).  Products over
 * a matrix with a split (sag_spmm_csr, sag_spmm_csr_t and the layers) take
 * two passes: the hub part into fp32 partial rows, whose gathers keep
 * hitting the same few rows of X and so are served from L2, then the cold
 * part with each row's partial added to its sum before the epilogue.  The
 * cold part may carry a split of its own (the next-busiest columns; the hub
 * part may not), so a chain of hub sets, each small enough for L2, takes one
 * pass each, every pass adding the previous partial rows to its own.  The
 * result differs from the one-pass product only by fp32 summation order.
 * The split pays on graphs with many entries per row, where the partial
 * rows cost little next to the gathers they speed up.
 *
 * col_slices: nonzero asks products over this matrix (sag_spmm_csr,
 * sag_spmm_csr_t, sag_spmm_csr_noalloc and the layers' SpMMs) whose rows of X
 * span more than 256 bytes to run as one pass per 128-byte column slice of
 * X (the last slice narrower), each pass writing its columns of Y with the
 * epilogue applied.  This is the column-block split of H in [CAGNET]'s 2D
 * and 3D algorithms ("Reducing Communication in Graph Neural Network
 * Training", the 2D section's block decomposition and the 3D section's
 * shorter, fatter pieces of H), run one block after another on one GPU:
 * every gather of a pass reads one cache line, so each L2 holds the lines of
 * as many times more rows of X as a whole row spans lines (four at 512-byte
 * rows), and on degree laws whose busiest columns carry much of the matrix
 * more of the gathers hit.  The price is
 * one more pass over the indices (and values) per slice and per-row work
 * repeated per slice, so whether it pays depends on the matrix (measured:
 * about 5% saved at 512-byte rows on a 2.45M-node power-law graph with 51
 * entries per row, 3-8% lost on some R-MAT matrices), and is best decided
 * by timing both on the matrix.  Rows of at most 256 bytes are always
 * gathered whole (two slices gain too little L2 reach for the second pass).
 * The result differs from the whole-row product only by fp32 summation
 * order.  Ignored by a matrix with a hub split (its passes take whole rows), by the
 * fused aggregate -> transform kernel and by GAT. */
typedef struct sag_csr {
    int64_t n_rows;
    int64_t n_cols;
    int64_t nnz;
    const int64_t* indptr;
    const int32_t* indices;
    const float* values;
    const int32_t* sched;
    int64_t n_short;
    int64_t n_medium;
    int64_t n_long;
    int64_t n_seg;
    int32_t seg_len;
    int32_t row_mean;
    const struct sag_csr* hub_part;
    const struct sag_csr* cold_part;
    int32_t col_slices;
} sag_csr;

/* ---------------------------------------------------------------------------
 * CSR build (setup, once per graph partition; synchronises `stream`).
 *
 * Builds, for the local row range [lo, hi) of an edge list over node ids
 * [0, n_global), the normalised adjacency A (n_local x (n_local + n_halo)),
 * optionally its transpose AT ((n_local + n_halo) x n_local), the degrees
 * and the HALO node list (Sylvie, "Graph Engine": the halo set of a
 * partition; DIGEST: the out-of-subgraph neighbours pulled from the stale
 * store).
 *
 * Steps: optional symmetrisation; input self-loops dropped; edges whose
 * destination lies outside [lo, hi) dropped; duplicates collapsed (A is
 * 0/1); optional self connections; halo_gid = ascending list of distinct
 * source ids outside [lo, hi); a local column c becomes c - lo, a halo
 * column n_local + its rank in halo_gid; each row sorted by column;
 * deg[r] = entries of local row r; deg[n_local + k] = deg_global[halo_gid[k]]
 * when deg_global is given, else 1 + (entries in halo column k); values per
 * `norm`; AT row c lists the rows r holding column c, ascending, with the
 * same values.
 *
 * src, dst : device int32[n_edges], edge src -> dst.
 * deg_global: nullable device int32[n_global].
 * Outputs (device, capacities in entries): indptr[n_local + 1];
 *   indices, values: cap_nnz entries; indptr_t[cap_halo + n_local + 1],
 *   indices_t, values_t: cap_nnz entries (all three NULL: no transpose);
 *   deg[n_local + cap_halo] (nullable); halo_gid[cap_halo] (nullable when
 *   no halo node appears).
 * *nnz and *n_halo (host) receive the true sizes.  If an id lies outside
 * [0, n_global) the call returns SAG_E_RANGE; if nnz > cap_nnz or n_halo >
 * cap_halo it returns SAG_E_WORKSPACE with the sizes set and outputs
 * unspecified.  Upper bounds: nnz <= (symmetrize ? 2 : 1) * n_edges +
 * n_local, n_halo <= n_global - n_local.
 */
size_t sag_csr_build_workspace_bytes(int64_t n_edges, int64_t n_global,
                                     int64_t lo, int64_t hi, unsigned flags);

/* Sizes of the build without its outputs (synchronises `stream`): the same
 * inputs, validation and first steps as sag_csr_build_normalize up to the
 * halo set, then *nnz and *n_halo (host) receive the entry count of A and
 * the number of halo nodes, so a caller can allocate outputs of exactly
 * that size.  Returns SAG_E_RANGE for an id outside [0, n_global) (the
 * sizes are then 0).  ws as for the build (the same size query). */
sag_status sag_csr_build_normalize_query(const int32_t* src, const int32_t* dst, int64_t n_edges,
                                         int64_t n_global, int64_t lo, int64_t hi, unsigned flags,
                                         int64_t* nnz /* host */, int64_t* n_halo /* host */,
                                         void* ws, size_t ws_bytes, void* stream);

sag_status sag_csr_build_normalize(const int32_t* src, const int32_t* dst, int64_t n_edges,
                                   int64_t n_global, int64_t lo, int64_t hi, unsigned flags,
                                   sag_norm norm, const int32_t* deg_global,
                                   int64_t cap_nnz, int64_t cap_halo,
                                   int64_t* indptr, int32_t* indices, float* values,
                                   int64_t* indptr_t, int32_t* indices_t, float* values_t,
                                   int32_t* deg, int32_t* halo_gid,
                                   int64_t* nnz /* host */, int64_t* n_halo /* host */,
                                   void* ws, size_t ws_bytes, void* stream);

/* Degree-binned schedule of a CSR (see sag_csr); synchronises `stream`.
 * seg_len: long-row segment length, a multiple of 64 in [64, 65536].
 * buf: device memory of sag_csr_schedule_bytes(A, seg_len) bytes, owned by
 * the caller and referenced by *A afterwards.  Fills the schedule fields of
 * *A (host struct). */
size_t sag_csr_schedule_bytes(int64_t n_rows, int64_t nnz, int32_t seg_len);
size_t sag_csr_schedule_workspace_bytes(int64_t n_rows);
sag_status sag_csr_schedule(sag_csr* A, int32_t seg_len, void* buf, size_t buf_bytes,
                            void* ws, size_t ws_bytes, void* stream);

/* Hub split of a CSR (setup, once per matrix; synchronises `stream`).
 * The product of a split matrix is the sum of the products of its parts:
 * the CAGNET page's 1D algorithm section sums the product block column by
 * block column; here a block is a group of the busiest columns (and, along
 * a chain, the next-busiest), so that its rows of X fit one L2.
 * The hub columns are the n_hub columns holding the most entries of A
 * (ties to the lower column id; all columns when n_hub >= n_cols).  Writes
 * two CSRs over A's rows and columns: the hub part (every entry of A in a
 * hub column) and the cold part (every other entry), each row's entries in
 * their order in A, values copied with them (values_* NULL when A has
 * none).  The caller wraps the arrays in two sag_csr structs (row_mean 0,
 * optionally scheduled with sag_csr_schedule) and attaches them to A's
 * hub_part and cold_part; nothing else of A changes.
 * Outputs (device, capacities in entries): indptr_hub, indptr_cold
 * [n_rows + 1]; indices_hub, values_hub [cap_hub]; indices_cold,
 * values_cold [cap_cold].  *nnz_hub (host) receives the hub part's entry
 * count (the cold part has nnz - *nnz_hub).  A part larger than its
 * capacity returns SAG_E_WORKSPACE with *nnz_hub set and outputs
 * unspecified; cap = nnz always suffices.  A with row_mean set must store
 * its values (the parts carry them).  ws: sag_csr_hub_split_workspace_bytes
 * bytes. */
size_t sag_csr_hub_split_workspace_bytes(int64_t n_rows, int64_t n_cols);
sag_status sag_csr_hub_split(const sag_csr* A, int64_t n_hub,
                             int64_t cap_hub, int64_t* indptr_hub, int32_t* indices_hub, float* values_hub,
                             int64_t cap_cold, int64_t* indptr_cold, int32_t* indices_cold, float* values_cold,
                             int64_t* nnz_hub /* host */, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Halo gather -- the DIGEST "pull": dst[k, :] = src[rows[k] - row_base, :]
 * for k < n, a bitwise row copy of d elements of type dt.  rows: device
 * int32[n] (typically the halo list of sag_csr_build_normalize, whose global
 * ids map to stale-buffer rows by subtracting row_base); rows[k] - row_base
 * must lie in [0, rows of src) (not checked).  src and dst must not overlap.
 */
sag_status sag_halo_gather(const void* src, int64_t ld_src, const int32_t* rows, int64_t row_base,
                           int64_t n, int64_t d, sag_dtype dt, void* dst, int64_t ld_dst,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Halo push -- the DIGEST "push" (DIGEST, system design: after an epoch a
 * partition stores its newly computed rows of its own nodes in the
 * representation store): dst[ids[k] - row_base, :] = src[k, :] for k < n,
 * a bitwise row copy.  With accumulate = 1 the rows are added instead,
 * dst += src in fp32 with one rounding to dt: the return of halo-node
 * gradients to their owner, which integrates them into its own rows
 * (Sylvie, "Backward Propagation").
 * src: [n, d] (ld_src); dst: [n_dst, d] (ld_dst); ids: device int32[n].
 * Targets outside [0, n_dst) are skipped.  Two equal targets in one call
 * race (the result is one of the writes, or an incomplete sum).  src and
 * dst must not overlap.  Asynchronous on `stream`.
 */
sag_status sag_halo_push(const void* src, int64_t ld_src, const int32_t* ids, int64_t row_base,
                         int64_t n, int64_t d, sag_dtype dt, int accumulate, void* dst,
                         int64_t ld_dst, int64_t n_dst, void* stream);

/* ---------------------------------------------------------------------------
 * Low-bit halo messages -- Sylvie's Quantizer and Dequantizer (Sylvie,
 * system overview, "Quantizer", "Communicator", "Dequantizer"; convergence
 * section, "Unbiased Low-bit Module").
 *
 * Each message row is one node feature vector h (finite values) quantized
 * to bits-bit codes (bits in {1, 2, 4, 8}; B = 2^bits - 1) with
 * zero = min(h), R = max(h) - min(h), scale = R / B, and per element
 * t = (h - zero) / scale, code = floor(t) + 1 with probability
 * t - floor(t), at most B (stochastic rounding; a row with R = 0 has all
 * codes 0; a subnormal R gives unspecified codes).  Each step is an fp32
 * operation rounded to nearest even, in that order.  The draw of element j
 * of stream id `node` in call `epoch`: Philox4x32-10 (Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
 * (j / 4, node, epoch, 0), key (seed & 0xffffffff, seed >> 32), the top 24
 * bits of word j % 4 times 2^-24 (the fp32 uniform on [0, 1)); code + 1
 * when the draw is below t - floor(t).  For every t >= 1/2 the code's
 * expectation is then exactly t (Sylvie, "Unbiased Low-bit Module").
 *
 * Codes: row k at codes + k * ld_codes (bytes); element j in bits
 * [bits*j, bits*j + bits) little-endian; codes must be 16-byte aligned and
 * ld_codes a multiple of 16 and >= sag_code_row_bytes(d, bits) (0 for bad
 * arguments).  Bits of elements >= d are written as 0 up to
 * ceil(d / 8) * bits bytes; the rest of a row is not touched.
 *
 * sag_quantize_rows: message row k quantizes src[rows[k]] (rows NULL:
 * src[k]) with stream id nodes[k] (nodes NULL: k); a row index outside
 * [0, n_src) gives an all-zero message row (codes, scale and zero 0).
 * scale, zero: device float[n].
 * sag_dequantize_rows: the recovered row zero[k] + code * scale[k] (fp32,
 * multiply then add, each rounded) goes to dst[ids[k] - row_base] (ids
 * NULL: dst[k]), or is added to it in fp32 when accumulate = 1 (the
 * gradient return); one rounding to dt.  Targets outside [0, n_dst) are
 * skipped.  Both calls are asynchronous on `stream`; inputs are caller-owned
 * device memory.
 */
size_t sag_code_row_bytes(int64_t d, int bits);
sag_status sag_quantize_rows(const void* src, int64_t ld_src, sag_dtype dt, const int32_t* rows,
                             int64_t n_src, const int32_t* nodes, int64_t n, int64_t d, int bits,
                             uint64_t seed, uint32_t epoch, uint8_t* codes, int64_t ld_codes,
                             float* scale, float* zero, void* stream);
sag_status sag_dequantize_rows(const uint8_t* codes, int64_t ld_codes, const float* scale,
                               const float* zero, int64_t n, int64_t d, int bits,
                               const int32_t* ids, int64_t row_base, int accumulate, sag_dtype dt,
                               void* dst, int64_t ld_dst, int64_t n_dst, void* stream);

/* ---------------------------------------------------------------------------
 * SpMM: Y = A X (CAGNET page: the aggregation A^T H of a layer, one output
 * row per CSR row; DIGEST: P_in H_in + P_out H~_out when X = [H_in ; H~_out]).
 * X: [A->n_cols, d] of type xt; Y: [A->n_rows, d] of type yt.  Supported
 * (xt, yt): (F32, F32), (BF16, BF16), (BF16, F32).  Accumulation is fp32;
 * d <= 1024 (fp32) or 2048 (bf16).
 * addend (nullable, type yt, ld ld_add): Y[r] += addend[r] for r < n_add,
 * added in fp32 before the single rounding to yt.
 * ws: sag_spmm_workspace_bytes(A, d) bytes (0 unless A has long rows).
 * sag_spmm_csr_t is the same operation, named for its use on the
 * transposed matrix in the backward pass (dH_ext = A_norm^T dZ).
 */
size_t sag_spmm_workspace_bytes(const sag_csr* A, int64_t d);
sag_status sag_spmm_csr(const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                        void* Y, int64_t ldy, sag_dtype yt,
                        const void* addend, int64_t ld_add, int64_t n_add,
                        void* ws, size_t ws_bytes, void* stream);
sag_status sag_spmm_csr_t(const sag_csr* AT, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                          void* Y, int64_t ldy, sag_dtype yt,
                          const void* addend, int64_t ld_add, int64_t n_add,
                          void* ws, size_t ws_bytes, void* stream);

/* SpMM for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same product as
 * sag_spmm_csr, with the same arguments but no workspace.  The long rows'
 * partial sums go into a fixed device array of sag_spmm_noalloc_scratch_bytes()
 * bytes (64 MiB) that the library holds on each GPU it runs on until the
 * process ends; the call allocates nothing, not even for tracing (it records
 * no trace events).  A matrix whose partials need more
 * (sag_spmm_workspace_bytes(A, d) above that size) returns SAG_E_WORKSPACE
 * before any launch.  Every call on one GPU shares that GPU's array, so
 * calls that overlap on one GPU (different streams, or threads) race; calls
 * ordered on one stream do not.  Nothing in the array needs clearing: each
 * call writes every partial it reads.  A matrix with a hub split is
 * multiplied here in one pass over its own arrays (its parts are not used),
 * so results are bitwise those of sag_spmm_csr on the same matrix without
 * the split. */
size_t sag_spmm_noalloc_scratch_bytes(void);
sag_status sag_spmm_csr_noalloc(const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                                void* Y, int64_t ldy, sag_dtype yt,
                                const void* addend, int64_t ld_add, int64_t n_add, void* stream);

/* ---------------------------------------------------------------------------
 * Layers.  In all four calls: dt is the storage type of activations,
 * activation gradients and W (F32 or BF16); accumulation is fp32; b, dW and
 * db are fp32.  W is row-major [w_rows, d_out] with ld = d_out (no
 * alignment needed).  n_local = A->n_rows; n_ext = A->n_cols = n_local +
 * n_halo; H_ext is [n_ext, d_in] (ld ldh): local rows first, then the halo
 * rows (e.g. from sag_halo_gather).  Y_pre (nullable) and Out are
 * [n_local, d_out] with ld ldo.
 *
 * Association order.  (A H) W = A (H W): the layer aggregates first when
 * d_in <= d_out and transforms first otherwise, so that the SpMM always
 * runs at the narrower width.  `save` holds what the backward pass needs
 * (the aggregate when aggregating first, nothing otherwise); its size is
 * sag_*_save_bytes and its content is private to the library.  The
 * backward call must get the same A^T, H_ext, W, save and sizes.
 *
 * Options (forward calls): a bit set; SAG_LAYER_FUSED asks for the fused
 * aggregate -> transform kernel (sag_aggregate_transform) where it applies
 * (the layer aggregates first and the widths fit); otherwise, and by
 * default (0), the separate SpMM and product run.  Both give the same
 * results up to fp32 summation order (the fused kernel reads A's own arrays,
 * so it takes no hub split into account).  Unknown bits return
 * SAG_E_INVALID.
 *
 * Widths.  The SpMM width min(d_in, d_out) is at most 1024 (fp32) or 2048
 * (bf16).  The dense products keep their weight slice in LDS, so the K of
 * each (d_in for the GCN forward, 2 d_in for a SAGE layer that aggregates
 * first, d_out or 2 d_out for the input-gradient products) must stay within
 * about 1024 fp32 / 2048 bf16 elements after padding to 128-byte chunks;
 * larger widths return SAG_E_UNSUPPORTED before any launch.
 */

enum { SAG_LAYER_FUSED = 1 };

/* GCN layer (CAGNET page, forward-propagation equation; Sylvie, "Forward
 * Propagation"):  Y = A H_ext W + b;  Out = relu ? max(Y, 0) : Y. */
size_t sag_gcn_save_bytes(int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt);
size_t sag_gcn_forward_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t d_out, sag_dtype dt);
sag_status sag_gcn_layer_forward(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                 const void* W, const float* b, int64_t d_out, int relu,
                                 unsigned options, sag_dtype dt, void* Y_pre, void* Out, int64_t ldo,
                                 void* save, size_t save_bytes,
                                 void* ws, size_t ws_bytes, void* stream);

/* GCN backward (CAGNET page: backpropagation uses the same SpMM and dense
 * products; Sylvie, "Backward Propagation": the halo rows of the input
 * gradient are what a partition sends back; DIGEST: the weight gradient
 * depends on the stale rows):
 *   G_Y = relu ? G_out * 1[Y > 0] : G_out   (ReLU'(0) = 0)
 *   dW = (A H_ext)^T G_Y  (fp32 [d_in, d_out], ld d_out)
 *   db = column sums of G_Y (fp32 [d_out], nullable)
 *   dH_ext = A^T G_Y W^T over AT ([n_ext, d_in], ld ldd, type dt;
 *            NULL skips it).
 * Y is the forward's Y_pre or its Out (same sign pattern; ld ldg, as G_out).
 * AT may be NULL only when dH_ext is NULL and the layer aggregates first. */
size_t sag_gcn_backward_workspace_bytes(const sag_csr* AT, int64_t n_local, int64_t d_in,
                                        int64_t d_out, sag_dtype dt);
sag_status sag_gcn_layer_backward(const sag_csr* AT, int64_t n_local,
                                  const void* H_ext, int64_t ldh, int64_t d_in,
                                  const void* W, int64_t d_out, int relu,
                                  const void* Y, const void* G_out, int64_t ldg,
                                  float* dW, float* db, void* dH_ext, int64_t ldd,
                                  sag_dtype dt, const void* save, size_t save_bytes,
                                  void* ws, size_t ws_bytes, void* stream);

/* GraphSAGE-mean layer (Sylvie, first section: the aggregate of the
 * neighbours' rows enters the update together with the node's own row;
 * mean aggregator, self first in the concatenation):
 *   M = A_mean H_ext;  Y = [H_local | M] W + b;  Out = relu ? max(Y,0) : Y.
 * W: [2 * d_in, d_out]; rows 0 .. d_in-1 act on the node's own row, the rest
 * on M.  A_mean is the CSR of sag_csr_build_normalize with the mean
 * normalisation; tagged row_mean, the forward reads only its pattern and
 * scales each row's sum by 1/len(r).  Any other CSR is used with its stored
 * values (a sum aggregator for SAG_NORM_NONE), in the forward and, through
 * its transpose, in the backward alike. */
size_t sag_sage_save_bytes(int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt);
size_t sag_sage_forward_workspace_bytes(const sag_csr* A_mean, int64_t d_in, int64_t d_out,
                                        sag_dtype dt);
sag_status sag_sage_layer_forward(const sag_csr* A_mean, const void* H_ext, int64_t ldh,
                                  int64_t d_in, const void* W, const float* b, int64_t d_out,
                                  int relu, unsigned options, sag_dtype dt, void* Y_pre, void* Out,
                                  int64_t ldo,
                                  void* save, size_t save_bytes,
                                  void* ws, size_t ws_bytes, void* stream);

/* GraphSAGE-mean backward:
 *   G_Y as for GCN;  dW = [H_local | M]^T G_Y (fp32 [2 * d_in, d_out]);
 *   db = column sums of G_Y (nullable);  [dH_self | dM] = G_Y W^T;
 *   dH_ext = A_mean^T dM over AT_mean, plus dH_self on the local rows
 *   ([n_ext, d_in], ld ldd; NULL skips it). */
size_t sag_sage_backward_workspace_bytes(const sag_csr* AT_mean, int64_t n_local, int64_t d_in,
                                         int64_t d_out, sag_dtype dt);
sag_status sag_sage_layer_backward(const sag_csr* AT_mean, int64_t n_local,
                                   const void* H_ext, int64_t ldh, int64_t d_in,
                                   const void* W, int64_t d_out, int relu,
                                   const void* Y, const void* G_out, int64_t ldg,
                                   float* dW, float* db, void* dH_ext, int64_t ldd,
                                   sag_dtype dt, const void* save, size_t save_bytes,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Fused aggregate -> transform (forward).  One kernel computes
 *   Z = A H_ext  (as sag_spmm_csr, rounded once to dt; stored when Z != NULL)
 *   Y = Z W + b                 (self = 0, the GCN layer's product)
 *   Y = [H_ext[:n_local] | Z] W + b   (self = 1, GraphSAGE: W is [2 d_in, d_out])
 *   Out = relu ? max(Y, 0) : Y  (Y_pre nullable, as for the layers)
 * with the sum of each 32-row tile kept in LDS and multiplied by W on the
 * matrix cores in the same kernel, so Z is not read back from HBM (the
 * CAGNET page's local SpMM followed by the product with W, in one pass).
 * dt, W, b, H_ext, Out and ld's as for the layers; Z is [n_local, d_in]
 * (ld ldz).  Supported: d_out <= 256 and d_in up to about 1000 bf16 / 500
 * fp32 elements (GraphSAGE: half that); else SAG_E_UNSUPPORTED before any
 * launch.  The GCN and GraphSAGE forward calls use it when given
 * SAG_LAYER_FUSED.  A row_mean CSR is summed over its pattern and each row
 * scaled, as in the separate SpMM.
 * ws: sag_aggregate_transform_workspace_bytes (16-B aligned). */
size_t sag_aggregate_transform_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t d_out,
                                               int self, sag_dtype dt);
sag_status sag_aggregate_transform(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                   const void* W, const float* b, int64_t d_out, int self,
                                   int relu, sag_dtype dt, void* Y_pre, void* Out, int64_t ldo,
                                   void* Z, int64_t ldz, void* ws, size_t ws_bytes, void* stream);
/* ---------------------------------------------------------------------------
 * Graph-attention layer.  The pages name GAT (Velickovic et al., 2018) among
 * the models that partitioned full-graph training serves (Sylvie, first
 * section and results table; DIGEST, evaluation section) without printing
 * its formulas; the layer is the paper's, with H heads of width d_head side
 * by side (head k owns columns [k d_head, (k + 1) d_head), F = H d_head):
 *   Wh = H_ext W;  x_vu = a_dst_k . Wh_k[v] + a_src_k . Wh_k[u] for each
 *   entry (v, u) of A;  e = LeakyReLU(x) with negative slope `slope`;
 *   alpha_v. = softmax of e_v. over row v;
 *   Y_k[v] = sum_u alpha_vu Wh_k[u] + b;  Out = relu ? max(Y, 0) : Y.
 * A's values are ignored (its pattern is the neighbourhood; build it with
 * SAG_SELF_LOOPS to include each node itself, SAG_NORM_NONE suffices).
 * dt as for the other layers; W is [d_in, F] (ld F); a_src, a_dst are fp32
 * [H, d_head]; b fp32 [F] (nullable).  Out is [n_local, F] (ld ldo).
 * `save` (sag_gat_save_bytes) keeps Wh, the per-head scores and the
 * softmax normalisers (nothing per entry) for the backward call.
 * Supported: 1 <= H <= 64, d_head a power-of-two number of 16-byte vectors
 * (8, 16, ..., 512 bf16; 4, ..., 256 fp32), F at most 2048 bf16 / 1024 fp32,
 * d_in within the transform's K limit; else SAG_E_UNSUPPORTED before any
 * launch.  A needs a schedule for power-law rows (as the SpMM). */
size_t sag_gat_save_bytes(int64_t n_local, int64_t n_ext, int64_t heads, int64_t d_head,
                          sag_dtype dt);
size_t sag_gat_forward_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t heads,
                                       int64_t d_head, sag_dtype dt);
sag_status sag_gat_layer_forward(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                 const void* W, const float* a_src, const float* a_dst,
                                 const float* b, int64_t heads, int64_t d_head, float slope,
                                 int relu, sag_dtype dt, void* Out, int64_t ldo,
                                 void* save, size_t save_bytes,
                                 void* ws, size_t ws_bytes, void* stream);

/* GAT backward: the gradients of <G_out, Out> by the chain rule through the
 * same steps (softmax derivative, LeakyReLU' = 1 where x > 0, else slope;
 * ReLU'(0) = 0):  dW fp32 [d_in, F] (ld F, nullable), da_src and da_dst fp32
 * [H, d_head] (nullable), db fp32 [F] (nullable), dH_ext [n_ext, d_in] (ld
 * ldd, type dt, nullable; its halo rows are what the partition returns to
 * their owners).  A and AT are the forward's matrix and its transpose (AT
 * from the same build); H_ext, W, a_src, a_dst, heads, d_head, slope, relu
 * and save must be the forward's.  Y (forward Out, ld ldg as G_out) gives
 * the ReLU mask. */
size_t sag_gat_backward_workspace_bytes(const sag_csr* A, const sag_csr* AT, int64_t d_in,
                                        int64_t heads, int64_t d_head, sag_dtype dt);
sag_status sag_gat_layer_backward(const sag_csr* A, const sag_csr* AT, const void* H_ext,
                                  int64_t ldh, int64_t d_in, const void* W, const float* a_src,
                                  const float* a_dst, int64_t heads, int64_t d_head, float slope,
                                  int relu, const void* Y, const void* G_out, int64_t ldg,
                                  float* dW, float* da_src, float* da_dst, float* db,
                                  void* dH_ext, int64_t ldd, sag_dtype dt,
                                  const void* save, size_t save_bytes,
                                  void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Dense building blocks of the layers, exported for tests and for callers
 * that compose their own layers.
 *
 * sag_gemm: C = [A1 | A2] B (+ bias) (+ addend), optionally ReLU, where A1
 * is [M, K1] (ld lda1), A2 is [M, K2] (ld lda2; K2 = 0 and A2 = NULL for a
 * single operand), B is [K1 + K2, N] row-major with ld ldb (trans_b = 0) or
 * given as its transpose [N, K1 + K2] with ld ldb (trans_b = 1); A1, A2, B,
 * addend and C have type dt; bias fp32[N]; C_pre (nullable) receives the
 * value before ReLU.  mask (nullable, [M, K1], ld ldmask, type dt)
 * multiplies A1 by 1[mask > 0] on load.
 * sag_gemm_tn: C = [A1 | A2]^T Bm (fp32 [K1 + K2, N], ld ldc) and
 * colsum = column sums of Bm (fp32[N], nullable), where Bm = B masked by
 * 1[mask > 0] when mask is given; A1, A2 have M rows; B, mask: [M, N].
 */
size_t sag_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt);
sag_status sag_gemm(int64_t M, int64_t N, const void* A1, int64_t lda1, int64_t K1,
                    const void* A2, int64_t lda2, int64_t K2,
                    const void* mask, int64_t ldmask,
                    const void* B, int64_t ldb, int trans_b, const float* bias,
                    const void* addend, int64_t ld_add, int relu,
                    void* C, void* C_pre, int64_t ldc, sag_dtype dt,
                    void* ws, size_t ws_bytes, void* stream);
size_t sag_gemm_tn_workspace_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt);
sag_status sag_gemm_tn(int64_t M, int64_t N, const void* A1, int64_t lda1, int64_t K1,
                       const void* A2, int64_t lda2, int64_t K2,
                       const void* B, int64_t ldb, const void* mask, int64_t ldmask,
                       float* C, int64_t ldc, float* colsum, sag_dtype dt,
                       void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement (opt-in, for benchmarks and profiling; not part of any
 * computation: results are the same with it on or off).  The switch and
 * the records belong to the calling host thread, so threads do not see each
 * other's.  While enabled, every internal operation (SpMM, dense product, mask,
 * packing of B, halo gather) records a pair of HIP events on its stream,
 * with its name and shape ("spmm[bf16,rows,nnz,d]", "gemm_nn[bf16,M,K,N]",
 * ...), its algorithmic bytes (each operand read once, each output written
 * once: for the SpMM 8 (rows + 1) + 8 nnz (4 nnz when no values are read)
 * + elt d (cols + rows), the epilogue's addend and Y_pre not counted) and
 * flops.
 * sag_trace_get synchronises on the record's stop event and returns its
 * elapsed milliseconds; name receives at most name_cap bytes including the
 * terminating NUL.  sag_trace_clear destroys the calling thread's records. */
sag_status sag_trace_enable(int on);
int64_t sag_trace_count(void);
sag_status sag_trace_get(int64_t i, char* name, size_t name_cap, float* ms, int64_t* bytes,
                         int64_t* flops);
sag_status sag_trace_clear(void);

/* Row-gather probe (measurement only): the rate at which the memory system
 * delivers the rows an SpMM over the same ids gathers, without its row
 * structure, values or epilogue.  Reads rows ids[0..n) of X (d elements of
 * type dt, row pitch ldx elements; every id must lie in [0, rows of X),
 * which is not checked) in order, in equal contiguous chunks of ids per
 * wavefront, with the SpMM's lane layout, and folds every 16-byte vector of
 * the rows' first ceil(d * elt / 16) vectors into per-lane sums of uint32
 * words (wrapping) written to sink.  sink: device memory of
 * sag_gather_probe_sink_bytes() bytes, 16-B aligned, owned by the caller;
 * summed over all its 16-byte entries, word k (0..3) equals the sum mod
 * 2^32 of word k of every such vector of every gathered row.  X and ldx * elt
 * must be 16-B aligned; rows wider than 4 KB return SAG_E_UNSUPPORTED.
 * Asynchronous on `stream`. */
size_t sag_gather_probe_sink_bytes(void);
sag_status sag_gather_probe(const void* X, int64_t ldx, int64_t d, sag_dtype dt, const int32_t* ids,
                            int64_t n, void* sink, size_t sink_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics. */
const char* sag_status_string(sag_status s);
const char* sag_last_error(void);   /* detail of the calling thread's last error */
const char* sag_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAG_H */
