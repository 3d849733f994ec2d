/*
 * kvc.h -- C ABI of libkvc.so: score-and-select compression of a prompt's KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * The path: for every KV head, the last w prompt queries (the observation
 * window) attend to the prefix keys; each attention row is softmax-normalised
 * over the prefix; the probabilities are averaged over the window into a
 * per-token importance (optionally with Keyformer's Gumbel noise and
 * temperature); ZigZag budgets may be allocated per layer from LMBA; each head
 * keeps its top-k tokens plus a recent window; K and V are gathered into a
 * compacted cache; ThinK may then prune key channels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless marked "host".  The library never
 *   allocates device memory on these paths and never frees caller memory; the
 *   caller owns every buffer, including the workspace (sized by the matching
 *   *_workspace_size function).  Inputs are read-only.
 * - Every call is enqueued on `stream` (a hipStream_t passed as void*; NULL
 *   means the null stream) and returns without synchronising.
 * - Arguments are validated on the host before anything is enqueued.  On
 *   KVC_E_ARG, KVC_E_SHAPE, KVC_E_WORKSPACE or KVC_E_UNSUPPORTED nothing is
 *   enqueued and the outputs are untouched.  A failed launch returns
 *   KVC_E_DEVICE.  Faults inside kernels surface at the caller's next
 *   synchronisation.  No C++ exception crosses this boundary.
 * - Tensors are row-major.  bf16 tensors are raw 16-bit patterns.  Element
 *   strides are in elements.  bf16 pointers and the strides between rows that
 *   the kernels read with 16-byte vectors must be 16-byte aligned / multiples
 *   of 8 elements (checked; KVC_E_ARG otherwise).
 * - Results are deterministic: the same inputs give the same bytes.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_E_ARG = 1,          /* invalid argument value or pointer                 */
  KVC_E_SHAPE = 2,        /* inconsistent sizes                                */
  KVC_E_WORKSPACE = 3,    /* workspace missing or smaller than required        */
  KVC_E_DEVICE = 4,       /* a HIP call or kernel launch failed                */
  KVC_E_UNSUPPORTED = 5   /* valid request the library does not implement      */
} kvc_status;

/* Static description of a status code; never NULL. */
const char* kvc_status_str(int status);

/* Version of this ABI (incremented on any incompatible change). */
int kvc_abi_version(void);

/* KV-cache size in bytes, 2 * B * S * L * N * D * elem_bytes: the size formula
 * of the ThinK page (papercache summary of arXiv 2407.21018), preliminaries on
 * KV-cache optimisation.  Returns -1 if an argument is negative or the product
 * overflows int64. */
int64_t kvc_cache_bytes(int64_t B, int64_t S, int64_t L, int64_t N, int64_t D, int64_t elem_bytes);

/* Channels kept per head by ThinK: T = floor((1 - lambda) * D) evaluated in
 * double (ThinK page, magnitude-based pruning).  Returns -1 unless
 * 0 <= lambda < 1 and D > 0. */
int kvc_think_channels(int D, double lambda);

/* ------------------------------------------------------------------------ */
/* kvc_score: observation-window importance.                                 */
/* ------------------------------------------------------------------------ */
/*
 * Computes, for each layer l, KV head g and prefix token j in [0, n), n = S - w,
 *
 *   x[h,i,j] = alpha_l * <Q_obs[l,h,i,:], K[l,g,j,:]>,      h in group g
 *   y        = x                          (gumbel == 0)
 *   y        = (x + zeta[h,i,j]) / tau    (gumbel != 0; tau = +inf gives y = 0)
 *   p[h,i,j] = exp(y[h,i,j] - max_j y[h,i,:]) / sum_j exp(...)   (over j < n)
 *   I[l,g,j] = sum_{h in group g} (1/w) sum_i p[h,i,j]
 *
 * Sources: ZigZagKV blog page (qidao123 thread 109074), SnapKV section (window
 * of the last prompt queries against the prefix, mean over the window's rows,
 * per head); ThinK page, query-driven pruning (softmax(Q K^T / sqrt(D)));
 * Keyformer blog page, Gumbel-distribution section (y = x + zeta with
 * zeta ~ Gumbel(0,1), then division by the temperature tau); KVzap news page,
 * architectural compression (grouped-query attention).
 * Grouping: G = H / Hkv query heads share one KV head, query head h reads KV
 * head floor(h / G), and a KV head's importance is the SUM of its G query
 * heads' window means (each row of I sums to G).
 * Noise (gumbel != 0): zeta = -ln(-ln u), u = (2*floor(X/2^9) + 1) * 2^-24,
 * X = word (j mod 4) of Philox4x32-10 (Salmon et al., SC'11) with key
 * (seed mod 2^32, seed >> 32) and counter (floor(j/4), S - w + i, h, 0).
 *
 * Layouts:
 *   q_obs      bf16, element (l,h,i,d) at l*q_layer_stride + h*q_head_stride + i*D + d
 *   k          bf16, element (l,g,j,d) at l*k_layer_stride + g*k_head_stride + j*D + d,
 *              rows j in [0, S) must be readable (only j < n are used)
 *   importance fp32 [L, Hkv, n] contiguous (written in full)
 *   layer_scales: NULL, or device fp32 [L] of alpha_l (then `scale` is ignored)
 * Errors: KVC_E_UNSUPPORTED unless D == 128; KVC_E_ARG unless L, H, Hkv,
 *   w >= 1, S >= 2, the four strides are multiples of 8, scale > 0 and finite
 *   (when layer_scales is NULL; the library cannot check a device array),
 *   tau > 0 (+inf allowed, NaN rejected) when gumbel != 0, and q_obs / k are
 *   16-byte aligned, importance 4-byte aligned; KVC_E_SHAPE unless
 *   H % Hkv == 0, 1 <= w < S, G * w <= 65536 (G = H / Hkv), L <= 65535,
 *   Hkv <= 65535, L * Hkv * ceil(n / 128) < 2^31, q_head_stride >= w*D, k_head_stride >= S*D and, for L > 1,
 *   q_layer_stride >= H*q_head_stride and k_layer_stride >= Hkv*k_head_stride;
 *   KVC_E_WORKSPACE if the workspace is missing, short or not 16-byte aligned.
 *   Up to 512 (Keyformer noise: 128) of a KV head's G*w query rows are staged
 *   on chip at a time; more rows are processed in chunks of that size.
 * Precision: bf16 products, fp32 accumulation and softmax statistics, fixed
 *   reduction order; relative error of I well under 1e-3.
 */
typedef struct kvc_score_args {
  int32_t L;                 /* layers scored by this call, >= 1                 */
  int32_t H;                 /* query heads                                      */
  int32_t Hkv;               /* KV heads                                         */
  int32_t w;                 /* observation window (last w prompt queries)       */
  int32_t S;                 /* prompt length                                    */
  int32_t D;                 /* head dimension (128)                             */
  int64_t q_head_stride;     /* elements between query heads (>= w*D)            */
  int64_t q_layer_stride;    /* elements between layers of q_obs                 */
  int64_t k_head_stride;     /* elements between KV heads (>= S*D)               */
  int64_t k_layer_stride;    /* elements between layers of k                     */
  float scale;               /* alpha when layer_scales == NULL (1/sqrt(D))       */
  const float* layer_scales; /* device [L] or NULL                                */
  int32_t gumbel;            /* 0: plain SnapKV scores; 1: Keyformer noise       */
  float tau;                 /* temperature (gumbel only), > 0, +inf allowed     */
  uint64_t seed;             /* Philox key (gumbel only)                         */
} kvc_score_args;

/* Workspace bytes kvc_score needs for these arguments (0 on invalid args). */
size_t kvc_score_workspace_size(const kvc_score_args* args /* host */);

kvc_status kvc_score(const kvc_score_args* args /* host */, const void* q_obs, const void* k,
                     float* importance, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_score_noalloc: kvc_score for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as kvc_score (bit-identical
 * importance), but the workspace is the library's static per-device scratch:
 * kvc_score_noalloc_max_workspace() bytes (16 MiB), held by every device the
 * library runs on until the process ends.  Neither this call nor its kernels
 * allocate or free memory.
 * Errors: as kvc_score; KVC_E_WORKSPACE, before any device call, when
 *   kvc_score_workspace_size(args) exceeds the scratch; KVC_E_ARG if `stream`
 *   belongs to a device other than the current one (the scratch used is the
 *   current device's); KVC_E_DEVICE if the scratch address of the current
 *   device cannot be obtained.
 * Concurrency: all calls on one device share its scratch, which keeps the last
 *   call's contents (every byte a call reads it has written first).  Calls
 *   that overlap in time on one device -- other streams, other host threads --
 *   race and corrupt each other's results; serialise them.
 */
size_t kvc_score_noalloc_max_workspace(void);

kvc_status kvc_score_noalloc(const kvc_score_args* args /* host */, const void* q_obs, const void* k,
                             float* importance, void* stream);

/*
 * kvc_score_causal: Keyformer's other reading of its prompt phase, a full
 * (causal) attention pass.  Window row i of query head h sits at position
 * P = S - w + i and sees the keys j <= P: x = alpha <q, k_j> (+ noise,
 * / tau, exactly as kvc_score, the noise counter using P), softmax over those
 * P + 1 keys, and I[l, g, j] = (1/w) sum over the rows of g's query heads of
 * p[row, j] for every j in [0, S) (0 from rows that cannot see j).  With
 * w = S every prompt position is a query.
 * Source: Keyformer blog page, closing paragraphs (the prompt phase is a full
 * attention pass, with the Gumbel noise, from which key tokens are picked).
 * Layout: as kvc_score, except importance fp32 [L, Hkv, S] and w <= S.
 * Errors: as kvc_score, plus KVC_E_SHAPE unless w <= S and w % 32 == 0.
 */
size_t kvc_score_causal_workspace_size(const kvc_score_args* args /* host */);

kvc_status kvc_score_causal(const kvc_score_args* args /* host */, const void* q_obs, const void* k,
                            float* importance, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_lmba_budget: ZigZag per-layer budgets from importance.                */
/* ------------------------------------------------------------------------ */
/*
 * For every layer l and KV head g: MBA[l,g] = the minimum m such that the m
 * largest entries of I[l,g,:] hold at least `mass` of the row's total.  Then
 * M_l = sum_g MBA[l,g] (LMBA_l = M_l / Hkv), R = total_budget - L*floor and
 *   B_l = floor + q_l,   q_l = floor(R*M_l / sum M) plus one unit for each of
 *   the R - sum q layers with the largest R*M_l mod sum M (ties: lower l),
 * in exact integer arithmetic; a layer above `capacity` is clamped to it and
 * the excess re-shared among the rest by the same rule.  If sum M == 0 every
 * layer weighs 1.
 * Sources: ZigZagKV blog page, section on ZigZagKV's new observations (MBA:
 * fewest KV entries keeping 90% of a head's attention; LMBA: mean over the
 * layer's heads) and section on ZigZag's space allocation (share of the total
 * budget proportional to LMBA, with a minimum reserved per layer).
 * Layout: importance fp32 [L, Hkv, n] contiguous, entries >= 0 (-0.0 counts
 *   as 0; NaN and negative entries are outside the contract).  mba int32
 *   [L, Hkv] or NULL; budgets int32 [L] (tokens per KV head, recent window
 *   included).  workspace: kvc_lmba_budget_workspace_size bytes when mba is
 *   NULL (it then holds the MBA), else unused.
 * Errors: KVC_E_ARG unless 1 <= L <= 1024, Hkv >= 1, n >= 1, 0 < mass <= 1,
 *   0 <= floor <= capacity, L*floor <= total_budget <= L*capacity and the
 *   pointers are non-null and 4-byte aligned; KVC_E_SHAPE if L*Hkv > 65535,
 *   total_budget >= 2^31 or Hkv*n >= 2^31; KVC_E_WORKSPACE if mba is NULL and
 *   the workspace is missing or short.
 * Arithmetic: each score x enters the MBA search as the 64-bit fixed-point
 *   integer floor(x * 2^s), s chosen per row so that n copies of the row's
 *   largest score fit in 62 bits; sums of these integers are exact and
 *   order-independent (bit-reproducible).  The truncation loses less than
 *   n * 2^-s of a row's total (about 1e-10 of its largest score at n = 16K),
 *   so only a crossing within that margin of mass * total can resolve
 *   differently from exact real arithmetic.  The target is ceil of the fp64
 *   product total * mass, clamped to the total (with mass = 1 the MBA is
 *   the number of scores whose fixed-point mass is nonzero).  The
 *   allocation is exact int64 arithmetic.
 */
size_t kvc_lmba_budget_workspace_size(int32_t L, int32_t Hkv, int32_t n);

kvc_status kvc_lmba_budget(const float* importance, int32_t L, int32_t Hkv, int32_t n, double mass,
                           int64_t total_budget, int32_t floor_per_layer, int32_t capacity,
                           int32_t* mba, int32_t* budgets, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_pool_importance: SnapKV 1D pooling of the importance.                 */
/* ------------------------------------------------------------------------ */
/*
 * For every row g (layer x KV head) and key j < n, with h = kernel / 2:
 *   KVC_POOL_AVG: out[g,j] = (1/kernel) * sum_{i=j-h}^{j+h} in[g,i], positions
 *                 outside [0, n) counting as 0 (zero padding);
 *   KVC_POOL_MAX: out[g,j] = max of in[g,i] over i in [j-h, j+h] and [0, n).
 * Source: ZigZagKV blog page, SnapKV section (the averaged scores are pooled
 * along the keys so the neighbours of a strong token are kept with it).  The
 * page gives no kernel size or type; kernel odd in [1, 255], stride 1.
 * Layout: fp32, row g at in + g*in_stride and out + g*out_stride (>= n when
 *   rows > 1); out must not alias in.  Sums run in a fixed order: the result
 *   is bit-reproducible.
 * Errors: KVC_E_ARG unless rows >= 1, n >= 1, kernel odd in [1, 255], mode
 *   KVC_POOL_AVG or KVC_POOL_MAX, in != out, both 4-byte aligned;
 *   KVC_E_SHAPE for a stride < n or rows > 65535.
 */
typedef enum kvc_pool_mode { KVC_POOL_AVG = 0, KVC_POOL_MAX = 1 } kvc_pool_mode;

kvc_status kvc_pool_importance(const float* in, int64_t in_stride, float* out, int64_t out_stride,
                               int32_t rows, int32_t n, int32_t kernel, int32_t mode, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_select_topk: per-head top-k plus the recent window.                   */
/* ------------------------------------------------------------------------ */
/*
 * Candidates C = [0, c), c = min(S - w, S - recent).  k_top = budget - recent.
 * Each head keeps the k_top candidates first in the order (importance
 * descending, position ascending) and every position of [S - recent, S);
 * the `budget` kept positions are written ascending.
 * Sources: ZigZagKV blog page, SnapKV section (per-head top-K by averaged
 * score, plus every token of the last window) and ZigZag's token-selection
 * section (the same with per-layer quotas); Keyformer blog page, prompt-phase
 * paragraph (w recent tokens plus k - w of the other n - w).
 * Layout: importance fp32, row g at importance + g * imp_head_stride (>= n =
 *   S - w entries, only the first c are read; entries must not be NaN);
 *   indices int32 [Hkv, budget] contiguous.
 * Errors: KVC_E_ARG unless 0 <= recent <= S, 1 <= w < S,
 *   recent <= budget <= c + recent.
 */
size_t kvc_select_topk_workspace_size(int32_t Hkv, int32_t n);

kvc_status kvc_select_topk(const float* importance, int64_t imp_head_stride, int32_t Hkv, int32_t S,
                           int32_t w, int32_t recent, int32_t budget, int32_t* indices,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvc_select_topk_layers: kvc_select_topk for L layers in one launch, with
 * per-layer budgets read on the device (the budgets kvc_lmba_budget writes),
 * so no host round trip sits between budgeting and selection.  Layer l keeps
 * budgets[l] tokens per KV head; its block of `indices` starts at
 * Hkv * (budgets[0] + ... + budgets[l-1]) and holds [Hkv, budgets[l]] (the
 * layout of per-layer calls on one flat buffer).
 * Source: as kvc_select_topk; ZigZagKV blog page, token-selection section
 * (each layer selects with its own quota).
 * Layout: importance fp32, row (l, g) at importance + l*imp_layer_stride +
 *   g*imp_head_stride; budgets int32 [L] on the device, each in
 *   [recent, c + recent] and summing to at most total_budget; indices int32
 *   with Hkv * total_budget entries.  A layer whose budget is out of range or
 *   whose block would pass Hkv * total_budget entries writes nothing.
 * Errors: as kvc_select_topk; KVC_E_UNSUPPORTED when c > 32768 (use one
 *   kvc_select_topk call per layer there).
 */
kvc_status kvc_select_topk_layers(const float* importance, int64_t imp_head_stride, int64_t imp_layer_stride,
                                  int32_t L, int32_t Hkv, int32_t S, int32_t w, int32_t recent,
                                  const int32_t* budgets, int32_t total_budget, int32_t* indices, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_select_threshold: keep every candidate scoring >= threshold.          */
/* ------------------------------------------------------------------------ */
/*
 * Candidates C = [0, c), c = min(S - w, S - recent), as for kvc_select_topk.
 * Head g keeps each candidate j with scores[g, j] >= threshold (compared in
 * fp32; a NaN score is never kept), ascending, then every position of
 * [S - recent, S).  The kept count varies per head and per prompt.  Heads are
 * packed: head g's positions are indices[offsets[g] .. offsets[g + 1]),
 * offsets[0] = 0, offsets[Hkv] = the total.
 * Source: KVzap news page, inference section (thresholding plus a sliding
 * window of recent tokens, giving a compression ratio that follows the
 * prompt's information density).
 * Layout: scores fp32, row g at scores + g * score_head_stride (>= S - w
 *   entries, only the first c read); indices int32 with room for
 *   Hkv * (c + recent) entries (the most that can be kept); offsets int32
 *   [Hkv + 1].  Both are written on the device; read offsets[Hkv] back to
 *   learn the total.
 * Errors: KVC_E_ARG unless 0 <= recent <= S, 1 <= w < S and threshold is not
 *   NaN (+-inf allowed); KVC_E_SHAPE if Hkv * (c + recent) >= 2^31.
 *   Integer sums only: the output is deterministic.
 */
size_t kvc_select_threshold_workspace_size(int32_t Hkv, int32_t S, int32_t w, int32_t recent);

kvc_status kvc_select_threshold(const float* scores, int64_t score_head_stride, int32_t Hkv, int32_t S,
                                int32_t w, int32_t recent, float threshold, int32_t* indices,
                                int32_t* offsets, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_compact: gather kept K/V rows into a dense cache.                     */
/* ------------------------------------------------------------------------ */
/*
 * k_out[g,t,:] = k[g, indices[g,t], :] and v_out likewise (raw bf16 bytes).
 * Source: Keyformer blog page, prompt-phase paragraph (the kept tokens form the
 * new, smaller cache); KVzap news page (cache of shape (2, L, H, T, D)).
 * Layout: k, v bf16, row j of head g at base + g*head_stride + j*D; k_out,
 *   v_out bf16 [Hkv, budget, D] contiguous.  v / v_out may both be NULL.
 *   D % 8 == 0, D <= 1024, budget * D / 8 < 2^31 (else KVC_E_SHAPE).  An
 *   index outside [0, S) yields a row of 0xFFFF (bf16 NaN) instead of a read
 *   out of bounds.
 */
kvc_status kvc_compact(const void* k, const void* v, int32_t Hkv, int32_t S, int32_t D,
                       int64_t k_head_stride, int64_t v_head_stride, const int32_t* indices,
                       int32_t budget, void* k_out, void* v_out, void* stream);

/*
 * kvc_compact_layers: kvc_compact for L layers in one launch with per-layer
 * budgets read on the device: layer l's block of `indices` and of the outputs
 * starts at row Hkv * (budgets[0] + ... + budgets[l-1]) and holds
 * [Hkv, budgets[l]] rows, k_out[row] = k[l, g, indices[row]] (v likewise).
 * Source: as kvc_compact, per layer (ZigZagKV's per-layer quotas).
 * Layout: k, v bf16, row j of head g of layer l at base + l*layer_stride +
 *   g*head_stride + j*D; budgets int32 [L] (device); indices int32 and
 *   k_out, v_out bf16 with Hkv * total_budget rows.  A layer whose block would
 *   pass Hkv * total_budget rows writes nothing; an index outside [0, S)
 *   yields a row of 0xFFFF.
 * Errors: as kvc_compact; KVC_E_UNSUPPORTED unless D / 8 divides 256;
 *   KVC_E_SHAPE if Hkv * L > 65535 or a layer stride is too small.
 */
kvc_status kvc_compact_layers(const void* k, const void* v, int32_t L, int32_t Hkv, int32_t S, int32_t D,
                              int64_t k_head_stride, int64_t k_layer_stride, int64_t v_head_stride,
                              int64_t v_layer_stride, const int32_t* budgets, int32_t total_budget,
                              const int32_t* indices, void* k_out, void* v_out, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_compact_ragged: gather kept rows of packed heads.                     */
/* ------------------------------------------------------------------------ */
/*
 * For each head g and each t in [offsets[g], offsets[g + 1]) ∩ [0, max_rows):
 * k_out[t, :] = k[g, indices[t], :] and v_out likewise (raw bf16 bytes): the
 * compressed cache of a selection whose kept count varies per head, packed
 * head after head as kvc_select_threshold writes it.
 * Source: as kvc_compact (the kept tokens form the new, smaller cache), with
 * the KVzap news page's variable per-prompt kept count.
 * Layout: k, v as for kvc_compact; indices int32 and offsets int32 [Hkv + 1]
 *   on the device (only the device reads them); k_out, v_out bf16
 *   [max_rows, D].  indices must hold max_rows entries.  Whatever offsets
 *   holds, no access leaves [0, max_rows) or [0, S) (an index outside [0, S)
 *   yields a row of 0xFFFF).
 * Errors: KVC_E_ARG for null or misaligned pointers, D % 8 != 0 or D > 1024;
 *   KVC_E_UNSUPPORTED unless D / 8 divides 256; KVC_E_SHAPE if
 *   max_rows * D / 8 >= 2^31.
 */
kvc_status kvc_compact_ragged(const void* k, const void* v, int32_t Hkv, int32_t S, int32_t D,
                              int64_t k_head_stride, int64_t v_head_stride, const int32_t* indices,
                              const int32_t* offsets, int32_t max_rows, void* k_out, void* v_out,
                              void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_channel_prune: ThinK key-channel pruning of a compacted cache.        */
/* ------------------------------------------------------------------------ */
/*
 * With U = the first budget - recent rows of each head of k_c (the non-recent
 * kept tokens, which precede the recent window): M[g,d] = (sum_{t in U}
 * |k_c[g,t,d]|^p)^(1/p); T = floor((1 - lambda) D); channels[g] = the T
 * channels first in the order (M descending, d ascending), written ascending;
 * mask[g,d] = 1 for kept channels, else 0; k_pruned[g,t,c] =
 * k_c[g,t,channels[g,c]] for t in U.  Recent rows keep all channels (they are
 * not copied).
 * Source: ThinK page, magnitude-based pruning (M = ||K[n,:,d]||_p, keep
 * T = floor((1-lambda) D), I = Top_T) and THINK's implementation (recent keys
 * unpruned, binary channel mask).
 * Layout: k_c bf16 [Hkv, budget, D] contiguous; channels int32 [Hkv, T];
 *   mask uint8 [Hkv, D] or NULL; k_pruned bf16 [Hkv, budget - recent, T].
 * Errors: KVC_E_ARG unless 0 <= recent <= budget, 0 <= lambda < 1, T >= 1,
 *   p in {1, 2}; D == 128 (else KVC_E_UNSUPPORTED).  Norms are fp32 sums in
 *   a fixed order.
 */
size_t kvc_channel_prune_workspace_size(int32_t Hkv, int32_t budget, int32_t D);

kvc_status kvc_channel_prune(const void* k_c, int32_t Hkv, int32_t budget, int32_t D,
                             int32_t recent, double lambda, int32_t p, int32_t* channels,
                             uint8_t* mask, void* k_pruned, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_channel_prune_query: query-driven ThinK key-channel pruning.          */
/* ------------------------------------------------------------------------ */
/*
 * As kvc_channel_prune with p = 2, except for the channel score.  A KV head g
 * is queried by the G query heads g*G .. g*G + G - 1; Q_g stacks their w
 * observation-window rows (G*w rows).  score[g,d] = ||Q_g[:,d] K_U[:,d]^T||_F,
 * which for the rank-1 outer product equals ||Q_g[:,d]||_2 ||K_U[:,d]||_2
 * (U as in kvc_channel_prune); the kernel ranks by the square of this
 * product, which orders channels the same way.  channels, mask and k_pruned
 * are then as for kvc_channel_prune.
 * Source: ThinK page, query-driven pruning (per-channel Frobenius norm of
 * Q[-S_obs:, d] K[:, d]^T, greedy top-T over channels), its observation-window
 * section (the last S_obs queries), and THINK's implementation (recent keys
 * unpruned, binary channel mask).
 * Layout: q_obs bf16, row r of query head h at q_obs + h*q_head_stride + r*D
 *   (q_head_stride in elements, a multiple of 8, >= w*D: the [H, w, D] tensor
 *   the scoring call reads); the rest as for kvc_channel_prune.
 * Errors: as kvc_channel_prune; KVC_E_ARG if q_obs is NULL or not 16-byte
 *   aligned, G < 1 or w < 1; KVC_E_SHAPE if Hkv*G > 65535 or q_head_stride is
 *   out of range.  fp32 sums in a fixed order.
 */
size_t kvc_channel_prune_query_workspace_size(int32_t Hkv, int32_t G, int32_t budget, int32_t D);

kvc_status kvc_channel_prune_query(const void* k_c, const void* q_obs, int32_t Hkv, int32_t G, int32_t w,
                                   int64_t q_head_stride, int32_t budget, int32_t D, int32_t recent,
                                   double lambda, int32_t* channels, uint8_t* mask, void* k_pruned,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* kvc_channel_prune_value: ThinK value-channel pruning.                     */
/* ------------------------------------------------------------------------ */
/*
 * U = the first budget - recent rows of each head (as for kvc_channel_prune).
 * Q_g stacks the w window rows of query heads g*G .. g*G + G - 1 (R = G*w
 * rows).  P = softmax over U of scale * Q_g K_c[g, U]^T (row-wise),
 * O = P V_c[g, U] ([R, D]), score[g, d] = ||O[:, d]||_2; channels[g] = the
 * T = floor((1 - lambda) D) channels first in the order (score descending, d
 * ascending), ascending; mask as for keys; v_pruned[g, t, c] =
 * v_c[g, t, channels[g, c]] for t in U.  Recent rows keep every channel.
 * Source: ThinK page, supplementary section on value-cache pruning (the
 * value-channel score ||softmax(Q[-S_obs:] K^T / sqrt(D)) V[:, j]||_F and
 * I = Top_T), with the observation window and THINK's implementation
 * (recent tokens unpruned, binary mask).  The page's scale is 1/sqrt(D).
 * Layout: k_c, v_c bf16 [Hkv, budget, D] contiguous; q_obs as for
 *   kvc_channel_prune_query; channels int32 [Hkv, T]; mask uint8 [Hkv, D] or
 *   NULL; v_pruned bf16 [Hkv, budget - recent, T].
 * Arithmetic: the softmax constants come from the scoring path's first pass
 *   (fp32, fixed-order folds); P is split into bf16 hi + lo for the P V MFMA
 *   (about 2^-17 relative), accumulated in fp32 and folded in a fixed order.
 * Errors: as kvc_channel_prune_query, plus KVC_E_ARG unless scale is finite
 *   and > 0 and v_c is 16-byte aligned; KVC_E_SHAPE if G*w > 65536.
 */
size_t kvc_channel_prune_value_workspace_size(int32_t Hkv, int32_t G, int32_t w, int32_t budget, int32_t recent,
                                              int32_t D);

kvc_status kvc_channel_prune_value(const void* k_c, const void* v_c, const void* q_obs, int32_t Hkv, int32_t G,
                                   int32_t w, int64_t q_head_stride, int32_t budget, int32_t D, int32_t recent,
                                   double lambda, float scale, int32_t* channels, uint8_t* mask, void* v_pruned,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Keyformer decode phase: score hand-over and one decode step.             */
/* ------------------------------------------------------------------------ */
/*
 * kvc_decode_init_scores: acc[g, t] = importance[g, indices[g, t]] when that
 * index is in [0, n) (a scored prefix token), else 0 (the prompt's window
 * tokens, which the prompt phase does not score).  The accumulated scores a
 * decode phase starts from.
 * Source: Keyformer blog page, closing paragraphs (the decode phase adds each
 * step's score to the score carried from before).
 * Layout: importance fp32, row g at importance + g * imp_head_stride (>= n
 *   when Hkv > 1); indices int32 [Hkv, budget]; acc fp32 [Hkv, budget].
 * Errors: KVC_E_ARG for negative sizes or null / misaligned pointers.
 */
kvc_status kvc_decode_init_scores(const float* importance, int64_t imp_head_stride, const int32_t* indices,
                                  int32_t Hkv, int32_t budget, int32_t n, float* acc, void* stream);

/*
 * kvc_keyformer_decode_step: one decode step of one layer.  The new token at
 * position t has query rows q[h] (h = g*G .. g*G + G - 1 for KV head g) and a
 * key and value per KV head.  For each KV head g it attends over the B cache
 * slots and itself: x_j = scale <q_h, k_j>, y_j = (x_j + zeta_j) / tau with
 * zeta_j the Keyformer Gumbel noise for query position t and key position
 * p_j (Philox4x32-10, key = seed, counter (p_j / 4, t, h, 0), word p_j mod 4,
 * as in kvc_score), tau = +inf giving y = 0; the step score of key j is the
 * sum over the G heads of softmax_j(y).  Every slot's acc grows by its step
 * score.  Among the slots with pos <= t - recent, the lowest (acc, pos) -- then
 * the lowest slot -- is evicted: the new token's key and value are written
 * there, pos = t, acc = the new token's step score, and evicted[g] = that slot
 * (-1 if no slot may leave; the cache then only accumulates).
 * Source: Keyformer blog page, Gumbel-distribution and temperature sections
 * (noisy tempered softmax as the score) and the closing paragraphs on the two
 * phases (decode on the reduced cache, the score accumulated over steps, the
 * w most recent tokens kept).
 * Layout: q bf16, row h at q + h * q_head_stride; k_new, v_new bf16 [Hkv, D];
 *   k_cache, v_cache bf16 [Hkv, B, D] (updated in place); pos int32 [Hkv, B]
 *   (distinct positions < t); acc fp32 [Hkv, B] (>= 0); evicted int32 [Hkv]
 *   or NULL.  The slots are unordered: only positions matter.
 * Arithmetic: fp32, reductions in a fixed order (bit-reproducible).  The
 *   workspace holds the step's logits and per-chunk softmax statistics
 *   (kvc_keyformer_decode_step_workspace_size bytes).
 * Errors: KVC_E_ARG unless 1 <= recent < B, t >= 0, scale finite and > 0,
 *   tau > 0 (+inf allowed), pointers non-null and aligned (16 bytes for the
 *   bf16 arrays and the workspace); KVC_E_UNSUPPORTED unless D == 128 and
 *   G <= 8; KVC_E_SHAPE for Hkv * G > 65535, B > 2^28 or a bad q stride;
 *   KVC_E_WORKSPACE for a missing or short workspace.
 */
size_t kvc_keyformer_decode_step_workspace_size(int32_t Hkv, int32_t G, int32_t B);

kvc_status kvc_keyformer_decode_step(const void* q, int64_t q_head_stride, const void* k_new, const void* v_new,
                                     void* k_cache, void* v_cache, int32_t* pos, float* acc, int32_t Hkv,
                                     int32_t G, int32_t B, int32_t D, int32_t t, int32_t recent, float scale,
                                     float tau, uint64_t seed, int32_t* evicted, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing (measurement support).                                      */
/* ------------------------------------------------------------------------ */
/*
 * While enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on its launch stream.  kvc_timing_read synchronises on
 * those events and reports, per kernel name, the number of launches and their
 * summed duration in milliseconds.  Enabling clears earlier records.  Not
 * thread-safe; meant for benchmarks, not for production paths.
 */
kvc_status kvc_timing_enable(int32_t enable);

/* Number of distinct kernel names recorded so far. */
int32_t kvc_timing_count(void);

/* Entry `idx` (0-based): name copied into name_buf (NUL-terminated, truncated
 * to name_len), launches and total milliseconds into *launches and *total_ms
 * (host pointers). */
kvc_status kvc_timing_read(int32_t idx, char* name_buf, int32_t name_len, int32_t* launches,
                           double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
