/*
 * kvq.h — C ABI of libkvq: blockwise entropy-constrained unbiased scalar
 * quantization (ECASQ) of KV-cache blocks at admission, on AMD MI355X
 * (gfx950).
 *
 * The method is the one of the page "Rate-adaptive KV-cache quantizer"
 * (synthcore idea 2502, after arXiv:2608.18147):
 *   - Implementation notes: the cache is cut into blocks (one head by 32
 *     tokens, or one head by a feature group); each block builds candidate
 *     codebooks from its minimum, maximum and quantiles; every candidate is
 *     scored by its distortion D_r and the entropy H_r of its expected symbol
 *     frequencies; one global multiplier lambda couples the blocks; the
 *     codebook, symbol stream and block lengths are stored; decoding happens
 *     before attention.
 *   - Mathematical statement / Key formulas (1)-(2): minimise sum_r D_r subject
 *     to sum_r d_r H_r <= B; for fixed lambda each block minimises
 *     D_r + lambda d_r H_r on its own.
 *   - Key formulas (3): unbiased stochastic interpolation between the two
 *     codepoints around x, conditional MSE (q_{i+1}-x)(x-q_i).
 *   - Key formulas (4): projected subgradient step on lambda.
 * The bisection on lambda follows the page "Joint Tucker-rank and
 * residual-bit KV allocator" (Mathematical statement: binary search on the
 * multiplier finds a budget-feasible allocation).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device memory owned by the caller.  The
 *     library's own state is one 8 KB pinned host buffer per calling thread
 *     (hipHostMalloc on first use, kept until the process ends) through
 *     which the synchronising calls read back their small results (for up to
 *     1024 grid-search blocks the solve's last kernel writes them into it
 *     directly); one 16 KB device buffer per calling thread and GPU for
 *     kvq_admit's one-launch decode admission (hipMalloc on its first such
 *     call, kept until the process ends); and the 60 KB static device
 *     scratch of kvq_admit_noalloc (one per GPU, part of the loaded code
 *     object).  No other device memory is allocated.  Sizes
 *     of every buffer come from kvq_plan (filled by kvq_plan_blocks).
 *   - Host pointers are marked "(host)".
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns KVQ_EINVAL or KVQ_ENOSPC and launches nothing.  Calls are
 *     asynchronous on the given stream (KVQ_OK means "enqueued"), except
 *     kvq_solve_lambda, which synchronises the stream to return lambda,
 *     the rate and the device status word (non-finite input found by
 *     kvq_eval_candidates is reported there as KVQ_ENONFINITE).
 *   - kvq_last_error() returns a thread-local text for the last failure.
 *   - Calls on different streams with different buffers are independent;
 *     a kvq_plan is immutable and may be shared between threads.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
#define KVQ_OK 0
#define KVQ_EINVAL (-1)      /* bad argument, shape, stride or pointer */
#define KVQ_EINFEASIBLE (-2) /* no lambda <= 2^64 meets the budget */
#define KVQ_ENONFINITE (-3)  /* NaN or Inf among the KV entries */
#define KVQ_ENOSPC (-4)      /* an output capacity is smaller than the plan needs */
#define KVQ_EHIP (-5)        /* HIP runtime error (launch, copy, sync) */

/* element types of KV tensors */
#define KVQ_F16 1
#define KVQ_F32 2

/* codebook search (kvq_block_spec.search) */
#define KVQ_GRIDS 0    /* {min,max} + uniform and quantile grids, k = 3..s */
#define KVQ_EXACT_DP 1 /* every endpoint-containing subset (2..s points) of a
                          quantile alphabet of alphabet_m points, exact DP */
#define KVQ_BEAM 2     /* the same alphabet and subsets, searched by a beam
                          over ordered codepoints (Implementation notes):
                          codebooks grow left to right with the DP's partial
                          cost; chains of equal length ending at the same
                          codepoint compete and the beam_width cheapest of
                          each group (ties: lexicographically smaller chain)
                          are extended; the best completed chain wins (ties:
                          shorter, then lexicographically smaller) */

/* multiplier update (kvq_solve_lambda.mode) */
#define KVQ_BISECT 0  /* bracket doubling then `iters` halvings; feasible end */
#define KVQ_SUBGRAD 1 /* choose at lambda_io, then one projected step */
#define KVQ_BISECT_GREEDY 2 /* KVQ_BISECT, then the greedy post-pass (grids) */

#define KVQ_MAX_TENSORS 2
#define KVQ_MAX_S 16
#define KVQ_MAX_BLOCK 4096
#define KVQ_MAX_ALPHABET 32
#define KVQ_MAX_BEAM 8

/* A KV tensor [outer, heads, tokens, dim] in device memory (caller-owned).
   Strides are in elements; every stride must be positive. */
typedef struct {
    const void* data;
    int32_t dtype; /* KVQ_F16 | KVQ_F32 */
    int32_t pad_;
    int64_t shape[4];
    int64_t stride[4];
} kvq_tensor;

/* Block shape and codebook search.  A block is one head by tokens_per_block
   tokens by dims_per_block features (Implementation notes). */
typedef struct {
    int32_t tokens_per_block; /* 32 for head x 32-token blocks */
    int32_t dims_per_block;   /* head_dim, or the feature-group width */
    int32_t s;                /* codebook size limit |Q| <= s, 2..16 */
    int32_t search;           /* KVQ_GRIDS | KVQ_EXACT_DP | KVQ_BEAM */
    int32_t alphabet_m;       /* KVQ_EXACT_DP / KVQ_BEAM alphabet size (2..32); else 0 */
    int32_t beam_width;       /* KVQ_BEAM: chains kept per group (1..8); else 0 */
} kvq_block_spec;

/* Result of kvq_plan_blocks: block geometry and the byte size of every buffer
   the other calls take.  Blocks are numbered tensor-major (tensor 0 first),
   then outer index, head, token chunk, feature group, all row-major; entries
   inside a block are row-major (token, then feature). */
typedef struct {
    int64_t n_blocks;      /* R */
    int64_t n_entries;     /* R * d_block */
    int32_t d_block;       /* d_r, entries per block (<= 4096) */
    int32_t n_cand;        /* GRIDS: candidates C = 1 + 2 (s - 2); EXACT_DP, BEAM: pairs */
    int32_t n_stats;       /* order statistics kept per block */
    int32_t s;
    int32_t search;
    int32_t alphabet_m;
    int32_t dtype;
    int32_t n_tensors;
    int32_t tokens_per_block;
    int32_t dims_per_block;
    int64_t tensor_blocks[KVQ_MAX_TENSORS]; /* blocks contributed by each tensor */
    int64_t shape[KVQ_MAX_TENSORS][4];      /* tensor shapes the plan was made for */
    size_t D_bytes;        /* kvq_eval_candidates D */
    size_t H_bytes;        /* kvq_eval_candidates H */
    size_t stats_bytes;    /* order statistics, fp32 [n_stats][R] (GRIDS) or [R][m] (EXACT_DP, BEAM) */
    size_t choice_bytes;   /* int32 [R] */
    size_t codebook_bytes; /* fp32 [R][s] */
    size_t m_bytes;        /* uint8 [R] */
    size_t offsets_bytes;  /* uint64 [R + 1] */
    size_t workspace_bytes;
    uint64_t max_code_words; /* code-stream words when every block uses s levels */
    int32_t rate_shift;    /* fixed-point scale 2^rate_shift of the rate sums */
    int32_t beam_width;    /* KVQ_BEAM: chains kept per group; else 0 */
} kvq_plan;

/* Human-readable name of a status code (static string). */
const char* kvq_status_string(kvq_status st);

/* Thread-local detail text of the last failing call ("" if none). */
const char* kvq_last_error(void);

/* Plan the block partition of n_tensors (1 or 2, same shape and dtype, e.g.
   K and V) tensors.  Host only: reads t[i].shape/stride/dtype (not data).
   Errors: KVQ_EINVAL when a tensor dimension is not a multiple of the block
   shape, the block has more than 4096 or fewer than 2 entries, s is outside
   2..16, the search mode or alphabet size is unknown, or shapes/dtypes of
   the tensors differ. */
kvq_status kvq_plan_blocks(const kvq_tensor* t, int32_t n_tensors,
                           const kvq_block_spec* spec, kvq_plan* out);

/* Score every candidate codebook of every block (Implementation notes; Key
   formulas (3); Mathematical statement for H_r).
   KVQ_GRIDS (candidate-major tables, so the solve's passes read them with
               coalesced loads):
               D[C][R]  (fp64) block distortion sum_t (q_{i+1}-x_t)(x_t-q_i),
               H[C][R]  (fp64) entropy in bits per entry of the expected
                        frequencies, candidates in the order {min,max},
                        U_3, E_3, ..., U_s, E_s;
               stats[n_stats][R] (fp32) order statistics at the sorted
                        distinct quantile ranks j (n-1)/(k-1) rounded half up
                        (first = minimum, last = maximum).
   KVQ_EXACT_DP and KVQ_BEAM: stats[R][alphabet_m] the alphabet order statistics (with
               repeats); with A the sorted distinct alphabet (m points) and
               pair p = index of (i < j) in row-major upper-triangle order of
               an alphabet_m-point alphabet, P = plan.n_cand =
               alphabet_m (alphabet_m - 1) / 2 pairs (pairs past the
               distinct points hold 0):
               D[R][P]      distortion of the entries in [A_i, A_j)
                            (closed at the last point) interpolated on A_i, A_j,
               H[R][P][2]   their masses sent to A_i and to A_j (entries).
   workspace: plan.workspace_bytes of device memory; its status word is
   reset here and set when an entry is NaN or Inf (reported by
   kvq_solve_lambda).  Asynchronous on stream s. */
kvq_status kvq_eval_candidates(const kvq_plan* p, const kvq_tensor* t, int32_t n_tensors,
                               double* D, double* H, float* stats,
                               void* workspace, hipStream_t s);

/* Choose every block's codebook under one multiplier (Key formulas (2),
   (4); bisection per the Tucker-allocator page).
   KVQ_BISECT: lambda = 0 if sum_r d_r H_r(argmin D) <= B sum_r d_r; else the
     bracket [0,1] doubles up to 2^64 until feasible, then `iters` halvings
     (iters <= 63); the feasible end is returned in *lambda_io (host).
   KVQ_BISECT_GREEDY: KVQ_BISECT, then the remaining budget is spent
     greedily (page "Joint Tucker-rank and residual-bit KV allocator",
     Implementation notes: swap candidates with the best distortion
     reduction per added bit): while some block has a candidate with more
     bits and less distortion whose added bits fit the remainder, the block
     with the largest (D_cur - D_c) / (d_r H_c - d_r H_cur) switches (ties:
     lowest block, then lowest candidate).  lambda is the bisection's;
     the rate returned is the filled one.  KVQ_GRIDS only.  Upgrades that
     fit the slack beyond the workspace pool: KVQ_ENOSPC.
   KVQ_SUBGRAD: blocks are chosen at *lambda_io (host, input); then
     *lambda_io <- max(0, lambda + eta (Rbar - B)) with Rbar the modelled
     bits per entry.
   Outputs (device): choice[R] (GRIDS: candidate index; EXACT_DP, BEAM: bitmask of
   the chosen distinct-alphabet points), codebook[R][s] (fp32, unused slots
   0), m[R] (levels), word_off[R+1] (exclusive scan of ceil(d_r w_r / 32),
   w_r = ceil(log2 m_r)); *rate_bits_per_entry_out (host) is the modelled
   rate sum_r d_r H_r / sum_r d_r of the choice.  Synchronises stream s at
   the end; KVQ_BISECT also waits once after the lambda = 0 probe, which
   decides whether the bracket passes are launched.
   workspace: the one kvq_eval_candidates wrote these tables with (its
   status word, the first 4 bytes, carries eval's NaN/Inf report and is
   read here); for tables from elsewhere, plan.workspace_bytes whose first
   4 bytes are zero (a zero-filled buffer will do).
   Errors: KVQ_ENONFINITE (from eval), KVQ_EINFEASIBLE, KVQ_EINVAL. */
kvq_status kvq_solve_lambda(const kvq_plan* p, const double* D, const double* H,
                            const float* stats, double B_bits_per_entry, int32_t mode,
                            int32_t iters, double eta, double* lambda_io,
                            double* rate_bits_per_entry_out, int32_t* choice,
                            float* codebook, uint8_t* m, uint64_t* word_off,
                            void* workspace, hipStream_t s);

/* kvq_solve_lambda with each block's distortion weighted: block r chooses
   argmin w_r D_r + lambda d_r H_r (the page's optional weighting of D_r by
   attention sensitivity, Implementation notes); the budget and the
   multiplier search are unchanged.  weight: device fp64 [R], finite and
   > 0 (other values give unspecified choices); NULL means every w_r = 1,
   i.e. exactly kvq_solve_lambda.  KVQ_GRIDS only (KVQ_EINVAL otherwise). */
kvq_status kvq_solve_lambda_weighted(const kvq_plan* p, const double* D, const double* H,
                                     const double* weight, const float* stats,
                                     double B_bits_per_entry, int32_t mode, int32_t iters,
                                     double eta, double* lambda_io,
                                     double* rate_bits_per_entry_out, int32_t* choice,
                                     float* codebook, uint8_t* m, uint64_t* word_off,
                                     void* workspace, hipStream_t s);

/* Unbiased stochastic interpolation of every entry on its block's codebook
   and fixed-width packing (Key formulas (3); Implementation notes).  The
   draw of entry t of block r is Philox4x32-10 with key (seed lo, seed hi),
   counter (t >> 2, r lo, r hi, 0), word t & 3, u = (word >> 8) 2^-24; the
   code is i+1 when u < p = (x - q_i)/(q_{i+1} - q_i), else i.  Every
   entry must lie in [q_0, q_{m_r - 1}] of its block's codebook, as it does
   for the codebooks kvq_solve_lambda writes (their end points are the
   block's minimum and maximum); the codes of entries outside it are
   unspecified.  Codes are a little-endian bit stream, block r starting at
   word word_off[r].
   codes_capacity_words must be >= plan.max_code_words (KVQ_ENOSPC).
   Asynchronous. */
kvq_status kvq_quantize_pack(const kvq_plan* p, const kvq_tensor* t, int32_t n_tensors,
                             const float* codebook, const uint8_t* m,
                             const uint64_t* word_off, uint64_t seed, uint32_t* codes,
                             uint64_t codes_capacity_words, hipStream_t s);

/* One admission step in one call: kvq_eval_candidates, kvq_solve_lambda and
   kvq_quantize_pack in that order on stream s, with the same arguments and
   results as the three calls (the page's admission: score the candidates,
   choose them under one multiplier, quantize; Key formulas (1)-(4)).  The
   codebooks and offsets the solve writes stay on the device, so the
   quantization is enqueued right behind it and the call waits once, at the
   end, for lambda, the modelled rate and the status (KVQ_BISECT also waits
   for its lambda = 0 probe).  For a decode loop this saves a host round trip
   per admitted batch.  mode: KVQ_BISECT or KVQ_SUBGRAD (KVQ_EINVAL
   otherwise).  On KVQ_ENONFINITE or KVQ_EINFEASIBLE the codes are written
   from the solve's placeholder result and have no meaning.  Errors: those of
   the three calls; arguments are all checked before anything is launched. */
kvq_status kvq_admit(const kvq_plan* p, const kvq_tensor* t, int32_t n_tensors, double* D,
                     double* H, float* stats, double B_bits_per_entry, int32_t mode,
                     int32_t iters, double eta, double* lambda_io,
                     double* rate_bits_per_entry_out, int32_t* choice, float* codebook,
                     uint8_t* m, uint64_t* word_off, uint64_t seed, uint32_t* codes,
                     uint64_t codes_capacity_words, void* workspace, hipStream_t s);

/* kvq_admit without a workspace argument and without any allocation, for
   callers that cannot allocate device or pinned memory (code under HIP graph
   capture, tight serving loops, harnesses that forbid hipMalloc).  The
   solve's workspace is a static device array of the library (60 KB per GPU,
   held by each GPU the library runs on until the process ends), so plans of
   at most 3,668,992 blocks are accepted (KVQ_ENOSPC beyond, with nothing
   launched).  Results are read back with a plain copy into the caller's host
   variables instead of the pinned staging buffer.  Arguments, outputs and
   errors are those of kvq_admit.  Every call on one GPU shares that GPU's
   scratch: calls that overlap in time on the same GPU (different streams or
   threads) race and give unspecified results; calls in sequence are
   independent (the scratch's stale contents are reset by the call's first
   kernels; the one-launch decode admission tags the words it publishes with
   a per-launch epoch, clears them when the epochs start over, and writes the
   header whole).  mode: KVQ_BISECT or KVQ_SUBGRAD. */
kvq_status kvq_admit_noalloc(const kvq_plan* p, const kvq_tensor* t, int32_t n_tensors, double* D,
                             double* H, float* stats, double B_bits_per_entry, int32_t mode,
                             int32_t iters, double eta, double* lambda_io,
                             double* rate_bits_per_entry_out, int32_t* choice, float* codebook,
                             uint8_t* m, uint64_t* word_off, uint64_t seed, uint32_t* codes,
                             uint64_t codes_capacity_words, hipStream_t s);

/* Decode before attention (Implementation notes): xhat[r][t] = Q_r[code_t]
   in fp32, blocks in plan order, entries row-major in the block.
   Asynchronous. */
kvq_status kvq_dequantize(const kvq_plan* p, const uint32_t* codes, const float* codebook,
                          const uint8_t* m, const uint64_t* word_off, float* xhat,
                          hipStream_t s);

/* ---- Entropy coding of the symbol stream (Implementation notes: the stored
   symbol stream is arithmetic-coded).  Each block's codes are rANS-coded
   (Duda, arXiv:1311.2540) with the block's own symbol counts as the model:
   k = ceil(log2 d_r), frequencies = counts with 2^k - d_r added to the most
   frequent symbol (lowest index among equals); 32-bit states in
   [2^16, 2^32), 16-bit words; 8 interleaved states, state i coding entries
   i, i + 8, ...; a block is f_0..f_{m_r - 1}, the 8 final states as (hi,
   lo), then the words emitted at steps 0, 1, ... (state order within a
   step), all 16-bit little-endian, zero-filled to a 32-bit boundary.  Block
   byte offsets (exclusive scan, R + 1 entries) are the stored block lengths. */

/* Buffer sizes for plan p (host only): the encoder's scratch and the
   largest possible coded stream, in bytes. */
kvq_status kvq_ans_sizes(const kvq_plan* p, uint64_t* scratch_bytes, uint64_t* stream_bytes);

/* Code the fixed-width codes of kvq_quantize_pack (codes, m, word_off as
   written by kvq_quantize_pack / kvq_solve_lambda).  scratch and stream are
   device buffers (4-byte aligned) of at least the kvq_ans_sizes bytes;
   block_off[R + 1] (device) receives the byte offset of each block in
   stream; *total_bytes_out (host) the stream's length.  Uses workspace's
   status word and scan area.  Synchronises stream s once.
   Errors: KVQ_ENOSPC (buffers smaller than kvq_ans_sizes, or a block
   outgrew its scratch region), KVQ_EINVAL. */
kvq_status kvq_ans_encode(const kvq_plan* p, const uint32_t* codes, const uint8_t* m,
                          const uint64_t* word_off, void* scratch, uint64_t scratch_bytes,
                          void* stream, uint64_t stream_bytes, uint64_t* block_off,
                          void* workspace, uint64_t* total_bytes_out, hipStream_t s);

/* Decode the coded stream and write each block's codepoints, fp32
   xhat[r][t] = codebook[r][symbol] (decode before attention).  stream and
   block_off as written by kvq_ans_encode (stream 4-byte aligned, else
   KVQ_EINVAL).  A block whose states do not end at 2^16 or whose words run
   out (a damaged stream) sets a bit in the workspace status word; reads
   stay inside the block's bytes.  Asynchronous on stream s. */
kvq_status kvq_ans_decode(const kvq_plan* p, const void* stream, const uint64_t* block_off,
                          const float* codebook, const uint8_t* m, float* xhat, void* workspace,
                          hipStream_t s);

/* ---- Decode attention over the quantized cache (Implementation notes:
   decode before attention; the decode runs inside the attention kernel, so
   only codes and codebooks are read).  For one new query per query head,
   o = sum_t softmax_t(scale q . k_t) v_t over every cached token, k_t and v_t
   the stored codepoints.  The plan must hold K (tensor 0) and V (tensor 1)
   [outer, heads, tokens, 128] cut into head x 32-token blocks; query head g
   reads KV head g / G, G = q_heads / heads any whole number >= 1 (run as
   passes over up to 4 query heads, each reading the codes once); K and V
   of equal shape, outer and heads at most 65535.  fp32 arithmetic. */

/* Bytes of the split-partials workspace for q_heads query heads (host). */
kvq_status kvq_decode_attention_workspace(const kvq_plan* p, int32_t q_heads, uint64_t* bytes);

/* codes, codebook, m, word_off: as written by kvq_solve_lambda and
   kvq_quantize_pack for plan p.  q: device fp32 [outer][q_heads][128];
   out: device fp32 [outer][q_heads][128]; work: device, at least the
   kvq_decode_attention_workspace bytes.  Asynchronous on stream s.
   Errors: KVQ_EINVAL (shape, group), KVQ_ENOSPC (workspace). */
kvq_status kvq_decode_attention(const kvq_plan* p, const uint32_t* codes, const float* codebook,
                                const uint8_t* m, const uint64_t* word_off, const float* q,
                                int32_t q_heads, float scale, float* out, void* work,
                                uint64_t work_bytes, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
