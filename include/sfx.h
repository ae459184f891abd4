/*
 * sfx.h -- C ABI of libsfx, the predictor-gated activation-sparse FFN step on
 * AMD Instinct MI355X (gfx950).
 *
 * One layer-step, as the PowerInfer page describes it (Method: per-layer predictor,
 * hybrid execution, neuron-aware operators) and as KAIROX extends it (Core method:
 * groups of 32 neurons, temporal activation momentum):
 *
 *   sfx_predict      scores = W2 relu(W1 x)                    per token
 *   sfx_compact      active = scores >= t, union over tokens,   ascending index list
 *   sfx_sparse_up    hact   = act(Wa[i] x + b_i) (ReLU / ReGLU) active rows only
 *   sfx_sparse_down  y      = sum_j hact_j Wd[idx_j]            active rows only
 *   sfx_tam_update   per-group momentum score and hot set       once per step, all layers
 *   sfx_hot_update   hot region slots + copy of entering groups  once per step, all layers
 *   sfx_select_kth, sfx_count_active, sfx_hot_first_order, sfx_gather_rows
 *                    offline calibration: thresholds, frequencies, hot-first order
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a caller-owned DEVICE pointer unless the comment
 *     says otherwise.  The library never frees or retains a pointer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call only enqueues kernels on it and returns: it never synchronises, never
 *     allocates device memory and reads no environment variables.  Calls may be
 *     captured into a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns a negative sfx_status and enqueues nothing.  SFX_E_LAUNCH
 *     reports a HIP launch error (hipGetLastError) after enqueueing.
 *   - Matrices are row-major and densely packed.  Device pointers must be 16-byte
 *     aligned (bit masks, index lists and counts: 4-byte aligned) and every row
 *     of a weight matrix must span a multiple of 16 bytes.
 *   - Workspaces must be 256-byte aligned, at least as large as the matching
 *     *_ws() query, and zero-filled before their first use; each call leaves the
 *     control words it uses at zero again or, where a call says so, in a state the
 *     next call continues from, except the sticky status words named below, which
 *     stay set until the caller clears them.  One workspace must not
 *     be used by two calls that may run at the same time.
 *   - Batch B (tokens per step) is 1..SFX_MAX_B.
 *   - The data passed to one call must not change until that call's kernels end.
 */
#ifndef SFX_H
#define SFX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFX_ABI_VERSION 2
#define SFX_MAX_B 64
#define SFX_MAX_GROUPS 1024
#define SFX_DOWN_SCRATCH_BYTES ((size_t)17 << 20)   /* static scratch of sfx_sparse_down_noalloc */

typedef enum {
  SFX_OK = 0,
  SFX_E_NULL = -1,        /* a required pointer is NULL */
  SFX_E_SHAPE = -2,       /* a size is out of range or inconsistent */
  SFX_E_DTYPE = -3,       /* unknown dtype / activation, or one the call does not take */
  SFX_E_ALIGN = -4,       /* a pointer or a row is not 16-byte aligned */
  SFX_E_WORKSPACE = -5,   /* workspace NULL, misaligned or smaller than the query */
  SFX_E_LAUNCH = -6,      /* HIP reported an error for an enqueued kernel */
  SFX_E_UNSUPPORTED = -7, /* the combination is valid but not built */
  SFX_E_DEVICE = -8,      /* no current HIP device could be queried */
  SFX_E_SCRATCH = -9      /* the shape needs more than the library's static scratch */
} sfx_status;

typedef enum {
  SFX_F32 = 0,   /* IEEE binary32 */
  SFX_F16 = 1,   /* IEEE binary16 */
  SFX_BF16 = 2,  /* bfloat16 (high half of binary32) */
  SFX_Q4G32 = 3  /* FFN rows only: symmetric int4, planar.  q [rows][cols/2] uint8,
                    byte c holds column 2c in its low nibble and 2c+1 in its high
                    nibble, two's complement in [-8, 7]; scales [rows][cols/32]
                    binary16, one per 32 consecutive columns; w = q * s. */
} sfx_dtype;

typedef enum {
  SFX_RELU = 0,  /* a = max(Wa_i . x + b_i, 0) */
  SFX_REGLU = 1, /* a = max(Wa_i . x + b_i, 0) * (Wl_i . x)  (gate = Wa, linear = Wl) */
  SFX_RELU2 = 2  /* a = max(Wa_i . x + b_i, 0)^2  (squared ReLU; sfx_sparse_up only) */
} sfx_act;

/* Host: static text for a status code. */
const char* sfx_status_str(int status);
/* Host: SFX_ABI_VERSION of the built library. */
int sfx_abi_version(void);

/* ---------------------------------------------------------------------------------
 * sfx_predict -- per-layer MLP predictor (PowerInfer page, Method, the predictor
 * pseudocode of §5.1: one hidden layer with ReLU, one score per FFN neuron).
 *
 *   hidden_b = max(W1 x_b, 0)   (fp32, kept in the workspace, never rounded to wdt)
 *   scores_b = W2 hidden_b      (fp32 accumulation)
 *
 *   wdt     SFX_F32, SFX_F16 or SFX_BF16: storage of x, W1 and W2.
 *   x       [B][d] wdt, the FFN input of each token.
 *   W1      [h][d] wdt.   W2 [f][h] wdt.  No biases.
 *   scores  [B][f] fp32, written.
 *   ws      >= sfx_predict_ws(wdt, B, d, h, f) bytes.
 * Rows: d*sizeof(wdt) and h*sizeof(wdt) must be multiples of 16 bytes.
 * From B = 3 on (fp16 / bf16) both layers run on the matrix cores; the second
 * takes the fp32 hidden as exact 16-bit pieces (two fp16 or three bf16 terms),
 * so scores keep fp32 accuracy.  With fp16 weights the hidden values must then
 * stay within 65504 in magnitude (the fp16 range of the leading piece); bf16
 * pieces cover the fp32 range.  Below 3 tokens (and for fp32 weights) there is no
 * such limit.
 * Workspace: a 256-byte control line, then (from 3 tokens) the pieces for 16, 32
 * or 64 tokens (B <= 16, <= 32, <= 64) and, when h / 16 is below 256, the first
 * layer's partial sums (its d walk is split over up to 4 workgroups per 16
 * rows) with one control word per 16 rows; below 3 tokens the fp32 hidden [B][h].
 * Word 0 of the control line is a sticky range flag: the matrix-core path sets it
 * nonzero when a hidden value is above 65504 (or NaN) with fp16 weights, and the
 * scores of that call are then wrong (inf / NaN terms).  The library never clears
 * it; the caller reads it after synchronising and writes zero to reset it.
 * ------------------------------------------------------------------------------- */
size_t sfx_predict_ws(int wdt, int B, int d, int h, int f);
int sfx_predict(void* stream, int wdt, int B, int d, int h, int f,
                const void* x, const void* W1, const void* W2,
                float* scores, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_predict_q4 -- the same predictor with int4 weights (PowerInfer page, Method,
 * §5.1; Pitfalls: the predictors are large -- for the OPT-30B-shaped layer at batch 1
 * an fp16 predictor is most of the bytes a step reads; int4 cuts it by 3.6x).
 *
 *   hidden_b = max(W1 x_b, 0) (fp32),  scores_b = W2 hidden_b,  W = q * s
 *
 *   x          [B][d] binary16.
 *   W1         [h][d/2] packed int4 codes, W1_scales [h][d/32] binary16 (the layout
 *              of SFX_Q4G32); W2 [f][h/2] codes, W2_scales [f][h/32].
 *   scores     [B][f] fp32, written.
 *   ws         >= sfx_predict_ws(SFX_Q4G32, B, d, h, f) bytes: the control line,
 *              then the fp32 hidden [B][h].
 * d and h must be multiples of 32; scale arrays 2-byte aligned.  Vector kernels at
 * every batch size (no fp16 range limit).
 * ------------------------------------------------------------------------------- */
int sfx_predict_q4(void* stream, int B, int d, int h, int f, const void* x,
                   const void* W1, const void* W1_scales, const void* W2, const void* W2_scales,
                   float* scores, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_compact -- threshold and compaction (PowerInfer page, Method, hybrid-execution
 * pseudocode: a neuron is computed when its score is >= the threshold; Paper vs code,
 * predictor threshold).  For B > 1 the active set is the union of the per-token sets.
 *
 *   scores     [B][f] fp32.  A NaN score is inactive.
 *   threshold  fp32 host scalar; compared as score >= threshold in fp32.
 *   tok_bits   [B][W] uint32 (W = ceil(f/32)) per-token masks, or NULL.
 *   union_bits [W] uint32 union mask.  Neuron i is bit (i % 32) of word i / 32;
 *              bits past f are zero.  Word g is group g of 32 neurons.
 *   idx        [kmax] int32: the union's neurons in ascending order in idx[0..count).
 *              Entries from count on are left unchanged.
 *   kmax       capacity of idx; must be >= f, so the list cannot overflow.
 *   count      device int32 scalar, written.  It stays on the device.
 *   ws         >= sfx_compact_ws(B, f) bytes (256 + 4 per 1024 neurons, rounded
 *              up to 256).  The workgroups hand their counts to each other through
 *              it, tagged with a 16-bit call counter kept in word 0 (carried from
 *              call to call, never cleared; zero-filling the whole workspace resets
 *              it), with bounded waits: a count that does not arrive within the bound
 *              sets word 1 of the workspace nonzero instead of hanging, and the list
 *              of that call is then undefined.  Word 1 is sticky: the library never
 *              clears it; the caller reads it after synchronising (nonzero = some
 *              call since the last reset timed out) and writes zero to reset it.
 * ------------------------------------------------------------------------------- */
size_t sfx_compact_ws(int B, int f);
int sfx_compact(void* stream, int B, int f, const float* scores, float threshold,
                uint32_t* tok_bits, uint32_t* union_bits, int32_t* idx, int kmax,
                int32_t* count, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_sparse_up -- gathered up (and gate) rows of the active neurons (PowerInfer page,
 * Method, neuron-aware operators of §5.4: only active rows are read; Paper vs code,
 * activation functions ReLU, ReGLU and squared ReLU).  Every token computes every
 * listed neuron.
 *
 *   hact[j][b] = act(Wa[idx[j]] . x_b + ba[idx[j]])      for j < *count, b < B
 *
 *   wdt      storage of the FFN rows: SFX_F32, SFX_F16, SFX_BF16 or SFX_Q4G32.
 *   act      SFX_RELU, SFX_REGLU or SFX_RELU2.
 *   x        [B][d] in wdt (binary16 when wdt = SFX_Q4G32).
 *   Wa       [f][d] activated branch, row = neuron (Q4: packed codes).
 *   Wa_scales Q4 scales [f][d/32] binary16, else NULL.
 *   ba       [f] fp32 bias of the activated branch, or NULL for none.
 *   Wl, Wl_scales  ReGLU linear branch, same layout as Wa; NULL for ReLU.
 *   idx, count     the list from sfx_compact (or any list of distinct neurons in
 *                  [0, f)); count is read on the device and clamped to kmax; an
 *                  index outside [0, f) yields a zero activation.
 *   hact     [kmax][B] fp32; rows j < count are written, the rest are unchanged.
 * Q4 requires d % 32 == 0.  From B = 3 on, fp16 / bf16 rows are multiplied on the
 * matrix cores (exact 16-bit products, fp32 sums).
 * ------------------------------------------------------------------------------- */
int sfx_sparse_up(void* stream, int wdt, int act, int B, int d, int f,
                  const void* x, const void* Wa, const void* Wa_scales, const float* ba,
                  const void* Wl, const void* Wl_scales,
                  const int32_t* idx, const int32_t* count, int kmax, float* hact);

/* ---------------------------------------------------------------------------------
 * sfx_sparse_down -- gathered neuron-major down rows (PowerInfer page, Method,
 * hybrid-execution pseudocode: y is the sum of the active neurons' contributions;
 * neuron-aware operators: blocks own disjoint neurons).
 *
 *   y[b][:] = sum_{j < count} hact[j][b] * Wd[idx[j]][:]
 *
 * The neurons are split into slices; each slice's partial sum goes to the
 * workspace and the last slice to finish a column tile adds the partials in slice
 * order, so y is bitwise reproducible.  y is overwritten (zero when count = 0).
 * From B = 3 on, fp16 / bf16 rows are multiplied on the matrix cores in fp32
 * (16x16x4 fp32 products, the activations used as they are).
 *
 *   Wd        [f][d] wdt, row = neuron (Q4: packed codes); Wd_scales as for Wa.
 *   idx, count, kmax, hact   as produced by sfx_compact / sfx_sparse_up.
 *   y         [B][d] fp32.
 *   ws        >= sfx_sparse_down_ws(wdt, B, d, kmax) bytes.
 * ------------------------------------------------------------------------------- */
size_t sfx_sparse_down_ws(int wdt, int B, int d, int kmax);
int sfx_sparse_down(void* stream, int wdt, int B, int d, int f,
                    const void* Wd, const void* Wd_scales,
                    const int32_t* idx, const int32_t* count, int kmax, const float* hact,
                    float* y, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_sparse_down_noalloc -- sfx_sparse_down for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments, same kernels, same y bit for bit, without `ws`.  The
 * partial tiles and tickets live in a static device array of the library, one per
 * GPU, of SFX_DOWN_SCRATCH_BYTES (17 MiB), held until the process ends; shapes
 * whose sfx_sparse_down_ws exceeds it return SFX_E_SCRATCH before anything is
 * enqueued (every fp16 / bf16 shape up to d = 8192 and 64 tokens fits).  The call allocates nothing (no hipMalloc, no library
 * allocation); the first call on a device looks up the array's address there.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (other streams, or concurrent host threads) race and give undefined y.
 * ------------------------------------------------------------------------------- */
int sfx_sparse_down_noalloc(void* stream, int wdt, int B, int d, int f,
                            const void* Wd, const void* Wd_scales,
                            const int32_t* idx, const int32_t* count, int kmax, const float* hact,
                            float* y);

/* ---------------------------------------------------------------------------------
 * sfx_dense_ffn -- the FFN over every neuron, without the predictor (PowerInfer page,
 * Implementation: long inputs switch to dense GPU computation in the prefill
 * stage; KAIROX page, Future work: choose sparse or dense kernels online from the
 * batch).  For every neuron i and token b:
 *
 *   hact[i][b] = act(Wa[i] x_b + b_i) (ReGLU: relu(.) (Wl[i] x_b); squared ReLU),
 *   y_b = sum_i hact[i][b] Wd[i]                                  (i ascending)
 *
 * It is what sfx_sparse_up / sfx_sparse_down compute for the list 0..f-1, with the
 * same kernels, so it equals the sparse step whose mask holds every neuron.  It
 * reads all rows of Wa (Wl) and Wd and no predictor weights: cheaper than the
 * sparse step once the union of the batch's masks holds most neurons.
 *   Arguments as sfx_sparse_up / sfx_sparse_down; hact [f][B] fp32 (written);
 *   ws >= sfx_dense_ffn_ws(wdt, B, d, f) bytes, 256-byte aligned, any contents.
 * ------------------------------------------------------------------------------- */
size_t sfx_dense_ffn_ws(int wdt, int B, int d, int f);
int sfx_dense_ffn(void* stream, int wdt, int act, int B, int d, int f, const void* x,
                  const void* Wa, const void* Wa_scales, const float* ba,
                  const void* Wl, const void* Wl_scales, const void* Wd, const void* Wd_scales,
                  float* hact, float* y, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_tam_update -- temporal activation momentum over groups of 32 neurons (KAIROX
 * page, Core method: item 3, decisions per group with at most 1024 groups per layer;
 * item 4, TAM with tau = (1 - lambda) + eps; item 6, set-difference update).
 * One call updates L layers (one workgroup each).
 *
 *   a_g   = (union_bits[l][g] != 0)                       group g touched this step
 *   s_g  <- lambda * s_g + (1 - lambda) * a_g              fp32
 *   cand  = { g : s_g > tau },  tau = (1 - lambda) + eps   in fp32
 *   topk  = first min(K, |cand|) of cand ranked by s desc, then g asc
 *   hot'  = topk;  entered = hot' & ~hot;  left = hot & ~hot'
 *
 *   L, G        layers, groups per layer (1..SFX_MAX_GROUPS).
 *   union_bits  [L][G] uint32: word g of layer l's union mask (sfx_compact output).
 *   lambda      in (0, 1); eps >= 0; K in 0..G.
 *   score       [L][G] fp32 state, in/out (start at zero).
 *   hot_bits    [L][ceil(G/32)] uint32 state, in/out (start at zero).
 *   entered_bits, left_bits  [L][ceil(G/32)] uint32, written.
 *   topk        [L][K] int32, written (entries past topk_count are -1).
 *   topk_count  [L] int32, written.
 *   ws          >= sfx_tam_ws(G, K) bytes (may be NULL when that is 0).
 * ------------------------------------------------------------------------------- */
size_t sfx_tam_ws(int G, int K);
int sfx_tam_update(void* stream, int L, int G, const uint32_t* union_bits,
                   float lambda, float eps, int K,
                   float* score, uint32_t* hot_bits, uint32_t* entered_bits,
                   uint32_t* left_bits, int32_t* topk, int32_t* topk_count,
                   void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_topk_now_update -- the reload rule TAM is compared with (KAIROX page,
 * Experiments: strategies and ablations, static TAM against Top-K): the hot set is
 * the groups most active in this step alone, with no memory of earlier steps.
 *
 *   n_g   = popcount(union_bits[l][g])                    neurons of g active now
 *   cand  = { g : n_g > 0 }
 *   topk  = first min(K, |cand|) of cand ranked by n desc, then g asc
 *   hot'  = topk;  entered = hot' & ~hot;  left = hot & ~hot'
 *
 * Arguments as sfx_tam_update without the score state (L, G, K, union_bits,
 * hot_bits, entered_bits, left_bits, topk, topk_count).  Same error behaviour.
 * ------------------------------------------------------------------------------- */
int sfx_topk_now_update(void* stream, int L, int G, const uint32_t* union_bits, int K,
                        uint32_t* hot_bits, uint32_t* entered_bits, uint32_t* left_bits,
                        int32_t* topk, int32_t* topk_count);

/* ---------------------------------------------------------------------------------
 * sfx_hot_update -- keeps the hot set's groups in a contiguous hot region of K group
 * slots per layer and copies only the groups that enter it (KAIROX page, Core
 * method: item 3, weights of co-active neurons stored together so that a group
 * moves as one contiguous block; item 4, the hot set fills the capacity; item 6,
 * only the set difference moves).  On one GPU the copy stands in for the reload a
 * CPU-GPU system pays, and its bytes measure the churn of the rule that chose the
 * hot set.  One call updates L layers:
 *
 *   1. each group g in left_bits frees its slot: group_of[slot_of[g]] = -1,
 *      slot_of[g] = -1;
 *   2. the free slots F (group_of[s] == -1), ascending, go to the groups E of
 *      entered_bits, ascending: slot_of[E_i] = F_i, group_of[F_i] = E_i, and
 *      copies[l][i] = {E_i, F_i}, for i < ncopies[l] = min(|E|, |F|);
 *   3. for every copy and every matrix m < nmat, group_bytes[m] bytes move from
 *      src[l][m] + E_i * group_bytes[m] to dst[l][m] + F_i * group_bytes[m].
 *
 * When entered_bits / left_bits come from one sequence of hot sets of at most K
 * groups (sfx_tam_update or sfx_topk_now_update with the same K), every entering
 * group finds a slot and group_of lists exactly the hot set.  Otherwise entering
 * groups past the free slots get slot -1 and no copy.
 *
 *   L, G, K        layers (1..1024), groups per layer (1..SFX_MAX_GROUPS), slots (1..G).
 *   entered_bits, left_bits  [L][ceil(G/32)] uint32 (bit g % 32 of word g / 32).
 *   slot_of        [L][G] int32 state, in/out (start at -1).
 *   group_of       [L][K] int32 state, in/out (start at -1).
 *   copies         [L][K][2] int32, written (entries past ncopies[l] untouched).
 *   ncopies        [L] int32, written.
 *   nmat           matrices per layer, 0..8 (0: slots only, no copy).
 *   group_bytes    host array [nmat]: bytes of one group in matrix m, a positive
 *                  multiple of 16 (at most 16 GiB summed over the matrices).
 *   src, dst       device arrays [L * nmat] of device pointers (16-byte aligned):
 *                  matrix m of layer l holds G groups (src) and K groups (dst).
 * ------------------------------------------------------------------------------- */
int sfx_hot_update(void* stream, int L, int G, int K,
                   const uint32_t* entered_bits, const uint32_t* left_bits,
                   int32_t* slot_of, int32_t* group_of, int32_t* copies, int32_t* ncopies,
                   int nmat, const size_t* group_bytes,
                   const void* const* src, void* const* dst);

/* ---------------------------------------------------------------------------------
 * Offline calibration (not part of the decode step).  PowerInfer page, Method:
 * offline profiling counts how often each neuron is active on calibration inputs,
 * and a neuron table maps the stored order to the model's; KAIROX page, Core
 * method, item 1: co-active neurons are stored as contiguous groups; Paper vs code,
 * predictor threshold: one threshold per layer.  A calibration pass runs
 * sfx_predict / sfx_compact on calibration tokens, then:
 *
 * sfx_count_active -- counts[i] += number of the B tokens whose mask holds neuron i.
 *   tok_bits [B][ceil(f/32)] uint32 (sfx_compact's per-token masks); counts [f]
 *   int32, in/out (start at zero).
 *
 * sfx_select_kth -- out[0] = the k-th smallest (0-based) of the n fp32 values, exact
 *   (a radix select on the values' order-preserving 32-bit keys; -0 sorts below
 *   +0, NaNs above +inf or below -inf by their sign).  With n = tokens x f scores
 *   and k = floor((1 - rho) n) it is the threshold at which a share rho of the
 *   calibration scores is active.  1 <= n < 2^32, k < n.  ws >= sfx_select_kth_ws()
 *   bytes, 256-byte aligned (any contents).  out: one device float.
 *
 * sfx_hot_first_order -- perm [f] int32, written: the hot-first neuron table, slot r
 *   of the new order holds old slot perm[r].  Neurons are ranked by
 *   (group count desc, group id asc, neuron count desc, slot asc), where the group
 *   count is the sum of counts over the group's members; group == NULL makes every
 *   neuron its own group (plain frequency order).  group [f] int32: group id of
 *   each slot in 0..f-1 (ids outside that range rank last, as group 0xFFFFFFFF with
 *   count 0); groups of exactly 32 members come out as aligned blocks of 32.
 *   ws >= sfx_hot_first_order_ws(f) bytes, 256-byte aligned, when group != NULL.
 *   1 <= f <= 2^24.
 *
 * sfx_gather_rows -- dst row r = src row idx[r] for r < n_dst (applies perm to a
 *   matrix, a bias or a scale table).  row_bytes a positive multiple of 4; src
 *   holds n_src rows; an idx entry outside 0..n_src-1 leaves its dst row
 *   untouched.  src and dst must not overlap.
 * ------------------------------------------------------------------------------- */
int sfx_count_active(void* stream, int B, int f, const uint32_t* tok_bits, int32_t* counts);
size_t sfx_select_kth_ws(void);
int sfx_select_kth(void* stream, size_t n, const float* values, size_t k, float* out,
                   void* ws, size_t ws_bytes);
size_t sfx_hot_first_order_ws(int f);
int sfx_hot_first_order(void* stream, int f, const int32_t* counts, const int32_t* group,
                        int32_t* perm, void* ws, size_t ws_bytes);
int sfx_gather_rows(void* stream, int n_dst, int n_src, size_t row_bytes, const void* src,
                    const int32_t* idx, void* dst);

/* ---------------------------------------------------------------------------------
 * sfx_ffn_step -- the whole step for L layers in one launch: for each layer in order,
 * exactly what sfx_predict, sfx_compact, sfx_sparse_up and sfx_sparse_down compute
 * (same outputs, same layouts), one layer after the other behind grid barriers.
 * Same passages as those four calls.  The data behind every layer's x must be in
 * place when the launch starts: a layer's x may not be an earlier layer's y of the
 * same launch (outputs are plain stores, visible to other compute units only once
 * the kernel has ended).
 *
 * One persistent workgroup per compute unit (the device must have 64, 128 or 256
 * of them, else SFX_E_UNSUPPORTED; workgroup w computes the scores of neurons
 * w + P j); phases are separated by grid
 * barriers in the workspace, so the grid must be resident on the device: the call
 * returns SFX_E_UNSUPPORTED when the occupancy query says one workgroup does not
 * fit on a compute unit, and kernels of other streams running at the same time
 * can still keep workgroups from starting.  A wait that does not complete within
 * its bound sets word 0 of the workspace nonzero instead of hanging, and the
 * outputs of that call are then undefined.  Word 0 is sticky: the library never
 * clears it, and while it is set the waits of later calls on the workspace give
 * up early (their outputs are undefined too).  The caller reads it after
 * synchronising and writes zero to reset it.
 *
 *   wdt      SFX_F16 or SFX_BF16 (x, predictor and FFN rows).  act: ReLU / ReGLU
 *            (squared ReLU returns SFX_E_UNSUPPORTED; sfx_sparse_up takes it).
 *   B        1..4.   d <= 4096, d and h multiples of 8, f <= 32768.
 *   L        number of layers; `layers` is a DEVICE array of L descriptors
 *            (caller-owned, unchanged until the kernel ends).  Each layer's idx
 *            holds at least f entries; tok_bits may be NULL; ba may be NULL.
 *   ws       >= sfx_ffn_step_ws(wdt, act, B, d, h, f) bytes, zero-filled before
 *            its first use, used on one device only.
 * Returns SFX_E_UNSUPPORTED for shapes the fused kernel is not built for; the
 * separate calls cover those.  Measured on MI355X against the separate calls (which
 * run on the matrix cores from 3 tokens): faster at 1 to 4 tokens on the OPT-6.7B and
 * LLaMA2-7B shapes (3 tokens, OPT-6.7B: 41.7 against 52.4 us per layer-step; 4
 * tokens, LLaMA2-7B: 49.6 against 55.5).
 * ------------------------------------------------------------------------------- */
typedef struct sfx_layer {
  const void* x;            /* [B][d] */
  const void* W1;           /* [h][d] */
  const void* W2;           /* [f][h] */
  const void* Wa;           /* [f][d] */
  const void* Wa_scales;    /* reserved, NULL */
  const float* ba;          /* [f] or NULL */
  const void* Wl;           /* [f][d] ReGLU linear branch, else NULL */
  const void* Wl_scales;    /* reserved, NULL */
  const void* Wd;           /* [f][d] neuron-major */
  const void* Wd_scales;    /* reserved, NULL */
  float threshold;
  int32_t reserved;
  float* scores;            /* [B][f] */
  uint32_t* tok_bits;       /* [B][ceil(f/32)] or NULL */
  uint32_t* union_bits;     /* [ceil(f/32)] */
  int32_t* idx;             /* [>= f] */
  int32_t* count;           /* device scalar */
  float* hact;              /* [>= f][B] */
  float* y;                 /* [B][d] */
  const void* xp;           /* [B][d] predictor input of sfx_ffn_pipeline (NULL = x);
                               sfx_ffn_step ignores it */
} sfx_layer;

size_t sfx_ffn_step_ws(int wdt, int act, int B, int d, int h, int f);
int sfx_ffn_step(void* stream, int wdt, int act, int B, int d, int h, int f, int L,
                 const sfx_layer* layers, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_ffn_pipeline -- the fused step with the predictor one layer ahead (KAIROX page,
 * Core method, item 2, Live Pipeline: the predictor of layer i + 1 runs on what is
 * known when layer i starts, overlapped with layer i's FFN; Key observation 1:
 * adjacent layers' hidden states have cosine similarity about 0.98).
 *
 * For each layer j, with its predictor input xp_j (descriptor field xp; NULL = x_j):
 *   scores_j = W2_j relu(W1_j xp_j);  idx_j = ascending {i : scores_j[b][i] >= t_j
 *   for some b};  hact = act(Wa_j[i] x_j + b_i);  y_j = sum_i hact Wd_j[i].
 * Outputs and layouts are those of sfx_ffn_step.  The kernel computes layer 0's
 * predictor first and then, while it gathers layer l's rows, layer l + 1's
 * predictor; a caller pipelining a real model passes xp_{l+1} = x_l (the input of
 * layer l, available when layer l starts) and, for layer 0, an input it has
 * before the step starts (e.g. layer 0's input of the previous token).  The data
 * behind every xp_j and x_j must be in place when the launch starts.
 * Same shapes, workspace, residency rule and sticky error word (word 0) as
 * sfx_ffn_step; shapes whose own-row scores or hidden staging do not fit the
 * kernel's LDS split return SFX_E_UNSUPPORTED (sfx_ffn_pipeline_ws returns 0).
 * ------------------------------------------------------------------------------- */
size_t sfx_ffn_pipeline_ws(int wdt, int act, int B, int d, int h, int f);
int sfx_ffn_pipeline(void* stream, int wdt, int act, int B, int d, int h, int f, int L,
                     const sfx_layer* layers, void* ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * sfx_stream_read -- measurement helper, not a step of the method.  Reads the nbytes
 * of buf once with 16-byte loads (2048 workgroups of 512 threads, 8 loads in flight
 * per thread) and writes 16384 uint32 checksums to out.  Its bandwidth is the
 * streaming-read ceiling that the step kernels' achieved HBM bandwidth is compared
 * with (PowerInfer page, Problem: batch-1 decode is bound by reading the weights).
 *   nbytes  a multiple of 16, >= 16.   buf 16-byte aligned.   out [16384] uint32.
 * ------------------------------------------------------------------------------- */
int sfx_stream_read(void* stream, const void* buf, size_t nbytes, uint32_t* out);

#ifdef __cplusplus
}
#endif
#endif /* SFX_H */
