/*
 * mla_verify.h -- C ABI of the MI355X (gfx950) speculative-verify attention
 * library for gated NoPE MLA with absorbed projections.
 *
 * What is computed (sources are the pages this library follows):
 *
 *  - "Kimi K3 support with DSpark speculative decoding", section "What does
 *    this PR do?": gated NoPE MLA with absorbed projections, and every decode
 *    step turned into a verify of k drafted tokens.  A request therefore
 *    brings a group of T = k+1 query tokens.  With absorption the per-head
 *    query lives in the 512-d latent space (q_latent = W_UK[h]^T q_nope) and
 *    attends directly over the compressed latent cache, which serves as both
 *    keys and values; W_UV is applied after the attention.
 *  - "Kimi K3: DSpark speculative decoding under Helix CP", first commit
 *    message ("Per-token primitive", "CuTe DSL MLA decode") and "Changes":
 *    each token of the group has its own attention bound kv_bounds[b, t] (the
 *    number of visible keys, its position + 1), which replaces the implicit
 *    causal bound; the softmax statistics are returned per token, and a token
 *    with no visible key yields the (-inf, 0) identity: lse = -inf, output 0.
 *    The third commit message of that page: such rows must never read pool
 *    bytes (a 0 * NaN would poison the merge).
 *  - Same page, commit on "fold_sq padding rows" and the reduction kernel:
 *    the group's tokens are folded into the head dimension, folded row
 *    r = t * H + h belongs to token r / H; padding rows clamp their token
 *    index and are never stored.
 *  - vLLM "specialized_decode.drafter.model", module docstring: the draft
 *    block's attention folds its tokens into heads (one decode row per
 *    request instead of one per token), and partial results are merged by an
 *    LSE combine followed by W_UV.
 *
 * Per request b, token t, head h, with L = clamp(kv_bounds[b,t], 0, P*64):
 *     s_j    = sm_scale * <q_latent[b,t,h,:], C_b[j,:]>        j < L
 *     lse    = ln sum_j exp(s_j)                    (-inf if L == 0)
 *     o_lat  = sum_j softmax(s)_j C_b[j,:]          (0    if L == 0)
 *     out    = sigmoid(gate[b,t,h,:]) * (W_UV[h] o_lat)   (gated entry)
 * where C_b[j] = latent_kv_pages[block_table[b, j/64], j%64, :], or, for an
 * fp8 cache, kv_scale times the value of that E4M3 code.
 *
 * fp8 latent cache (kv_dtype = MLA_KV_FP8_E4M3).  The first page serves with
 * an fp8 KV cache ("--kv-cache-dtype fp8" in its launch command), and the
 * Helix page notes that its per-token-bound decode kernel still rejects fp8
 * KV.  Neither fixes the encoding, so this library reads it as OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * 0x7F / 0xFF are NaN) with one scale per cache: a latent element is
 * kv_scale * value(code), for its use as key and as value alike.  Queries,
 * softmax weights and outputs stay as in the bf16 path.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major, contiguous, with
 *    the shapes given below, and 16-byte aligned.  bf16 is stored as its
 *    16-bit pattern (mla_bf16), fp8 as its 8-bit code.
 *  - The caller owns every buffer and the stream.  The library never
 *    allocates, frees or keeps a pointer after it returns; inputs are
 *    read-only; outputs are fully overwritten (masked rows get 0 / -inf).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  They do no host synchronisation and no device->host copy,
 *    so they may be captured into a hipGraph.
 *  - Results are deterministic: identical inputs give identical bits.
 *  - Return value: MLA_OK (0) or a negative MLA_ERR_* code.  Argument
 *    checks run on the host before any HIP call; unsupported requests fail
 *    loudly and never fall back to another path.
 *  - Device-side preconditions (documented, checked defensively):
 *    kv_bounds values are clamped into [0, max_pages_per_req * 64];
 *    block_table[b, p] must lie in [0, num_pool_pages) for every page p
 *    below ceil(max_t bound / 64) -- other entries are never read, and an
 *    out-of-range id is not dereferenced (its keys then read as zeros, an
 *    undefined but fault-free result); pool slots past a request's largest
 *    bound may hold any bytes, NaN included.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t mla_bf16; /* bf16 bit pattern, round-to-nearest-even */

enum mla_verify_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL                  */
  MLA_ERR_SHAPE = -2,       /* latent != 512, page != 64, T/H/B out of range */
  MLA_ERR_DTYPE = -3,       /* kv_dtype not MLA_KV_BF16 / MLA_KV_FP8_E4M3, */
                            /* or fp8 where the entry point takes bf16 only */
  MLA_ERR_ARG = -4,         /* bad sm_scale, num_splits, pool size, or a   */
                            /* pointer that is not 16-byte aligned         */
  MLA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required  */
  MLA_ERR_DEVICE = -6,      /* no GPU visible, or the current one is not gfx950 */
  MLA_ERR_HIP = -7          /* a HIP call or kernel launch failed          */
};

enum mla_verify_kv_dtype {
  MLA_KV_BF16 = 0,
  MLA_KV_FP8_E4M3 = 1       /* OCP FP8 E4M3 codes times kv_scale           */
};

/* Limits (MLA_ERR_SHAPE outside them). */
#define MLA_VERIFY_LATENT 512
#define MLA_VERIFY_PAGE 64
#define MLA_VERIFY_NOPE 128       /* per-head value dim of W_UV / gate / out */
#define MLA_VERIFY_MAX_Q_LEN 16
#define MLA_VERIFY_MAX_HEADS 128
#define MLA_VERIFY_MAX_SPLITS 64
/* Balanced-chunk partition (mla_verify_attn_partials): the start-up cost of
 * one (request, chunk) item, counted in 32-key units of key-loop time. */
#define MLA_VERIFY_ITEM_UNITS 6
/* Device scratch behind mla_verify_attn_gated_noalloc (64 MiB per GPU). */
#define MLA_VERIFY_STATIC_SCRATCH_BYTES (64u << 20)

typedef struct mla_verify_params {
  int32_t batch;             /* B >= 1 requests                              */
  int32_t q_len;             /* T = k+1 tokens per group, 1..16              */
  int32_t num_heads;         /* H, 1..128                                    */
  int32_t latent_dim;        /* must be 512                                  */
  int32_t page_size;         /* must be 64                                   */
  int32_t max_pages_per_req; /* P, block_table row stride (>= 1)             */
  int32_t num_pool_pages;    /* N, pages in latent_kv_pages (>= 1)           */
  int32_t num_splits;        /* 0 = library's choice; 1..64 = forced split-KV */
  float sm_scale;            /* softmax scale, finite and > 0                */
  int32_t kv_dtype;          /* MLA_KV_BF16 or MLA_KV_FP8_E4M3 (attention
                                entry points; the cache updates take bf16)  */
  int32_t tile_rows;         /* 0 = library's choice; 32, 64 or 128 = forced
                                folded rows per attention workgroup          */
  float kv_scale;            /* fp8 cache: latent = kv_scale * value(code),
                                finite and > 0; ignored for bf16            */
} mla_verify_params;

/* Validates `p` (pure host code, no HIP call).  MLA_OK or an error code. */
int mla_verify_check(const mla_verify_params* p);

/* The number of KV splits S the library will use for `p` (resolves
 * num_splits == 0).  Pure host code.  Returns S >= 1, or an error code. */
int mla_verify_num_splits(const mla_verify_params* p, int gated);

/* The folded rows per attention workgroup (32, 64 or 128) the library will
 * use for `p` (resolves tile_rows == 0).  Pure host code.  Returns the tile
 * rows, or an error code. */
int mla_verify_tile_rows(const mla_verify_params* p, int gated);

/* Workspace bytes the call needs (0 when it needs none).  `gated` selects
 * mla_verify_attn_gated.  Pure host code.  Layout: normalised partial
 * outputs [S][B*T*H][512] in bf16, then partial LSEs [S][B*T*H] in fp32.
 * Returns MLA_OK or an error code; *bytes is written only on success. */
int mla_verify_workspace_size(const mla_verify_params* p, int gated, size_t* bytes);

/* Verify attention, latent output ("Kimi K3: DSpark speculative decoding
 * under Helix CP", first commit message, "Per-token primitive": attention
 * over the paged latent cache with one bound per query token, returning the
 * per-token LSE, and the (-inf, 0) identity for a token with no visible key;
 * the group's tokens folded into the head dimension as in the vLLM drafter
 * page's module docstring).
 *   q_latent        [B, T, H, 512] bf16   absorbed queries (row t*H+h = fold)
 *   latent_kv_pages [N, 64, 512]   bf16   paged latent cache (fp8 E4M3
 *                                         codes, 512 B per key row, when
 *                                         kv_dtype is MLA_KV_FP8_E4M3)
 *   block_table     [B, P]         int32  page ids in logical order
 *   kv_bounds       [B, T]         int32  visible-key count per token
 *   out_latent      [B, T, H, 512] bf16   o_lat (0 for rows with bound 0)
 *   lse             [B, T, H]      fp32   natural-log LSE (-inf if bound 0)
 *   workspace       mla_verify_workspace_size(p, 0) bytes, or NULL if 0
 * Errors: MLA_ERR_NULL/SHAPE/DTYPE/ARG/WORKSPACE (host), MLA_ERR_DEVICE,
 * MLA_ERR_HIP (launch failure, reported without synchronising). */
int mla_verify_attn(const mla_verify_params* p,
                    const mla_bf16* q_latent,
                    const void* latent_kv_pages,
                    const int32_t* block_table,
                    const int32_t* kv_bounds,
                    mla_bf16* out_latent,
                    float* lse,
                    void* workspace, size_t workspace_bytes,
                    void* stream);

/* The attention half of mla_verify_attn on its own: the S = mla_verify_num_splits(p, 0)
 * split-KV results, for a caller that merges them itself, for example after
 * exchanging them between ranks that hold different pages of one request
 * ("Kimi K3: DSpark speculative decoding under Helix CP", "Changes": each
 * context-parallel rank returns its partial output with its softmax
 * statistics, and a rank with no visible key returns the (-inf, 0) identity).
 *   part_o    [S, B*T*H, 512] bf16  split s's output, normalised by split s's
 *                                   own softmax sum; rows whose split sees no
 *                                   key are left unwritten
 *   part_lse  [S, B*T*H]      fp32  split s's natural-log LSE (-inf: no key)
 * Partition: the folded rows of a request are processed in tiles of
 * tr = mla_verify_tile_rows(p, 0) rows (the last tile of a request may be
 * partial); a tile sees the keys below L, the largest bound among the tokens
 * of its rows.
 *  - Tiles of 128 rows (bf16 or fp8 cache) with S >= 2, B <= 2000 and P <= 1024
 *    (balanced chunks): request b has U_b = ceil(n_b / 32) units of 32 keys, n_b its
 *    largest bound, and occupies V_b = U_b + F positions (F =
 *    MLA_VERIFY_ITEM_UNITS; V_b = 0 when U_b = 0): F for its start-up, then
 *    its units.  The requests laid end to end (request b at position
 *    st_b = V_0 + ... + V_(b-1), V positions in all; its units at
 *    positions st_b + F ...) are cut into chunks of C = max(ceil(V / g),
 *    ceil(2 P / (S - 1))) positions, g = 8 * floor(32 / (tiles per
 *    request)); the last chunk runs to the end.  Slot j of request b covers
 *    the units of chunk floor((st_b + F) / C) + j that belong to it, as
 *    request keys [32 a, 32 a') (each tile clips them to its own L); its
 *    slots past its last chunk are empty (lse = -inf).
 *  - Otherwise a tile's n = ceil(L / 64) pages go to S' = min(S, ceil(n / m))
 *    contiguous splits, split s < S' holding pages [floor(s n / S'),
 *    floor((s+1) n / S')), with m = max(1, floor(ceil(P / S) / 2)); splits
 *    s >= S' are empty (lse = -inf).  For a batch of similar lengths S' = S;
 *    a short request in a ragged batch takes fewer splits.
 * Combining: lse = ln sum_s exp(lse_s), out = sum_s exp(lse_s - lse) part_o_s
 * (mla_verify_lse_combine).  Errors as mla_verify_attn. */
int mla_verify_attn_partials(const mla_verify_params* p,
                             const mla_bf16* q_latent,
                             const void* latent_kv_pages,
                             const int32_t* block_table,
                             const int32_t* kv_bounds,
                             mla_bf16* part_o,
                             float* part_lse,
                             void* stream);

/* LSE combine ("Kimi K3: DSpark speculative decoding under Helix CP",
 * "Changes": partial results merged through their softmax statistics, with
 * (-inf, 0) as the identity).  rows = B*T*H, num_splits = S in 1..64;
 * layouts as mla_verify_attn_partials; writes out_latent [rows, 512] bf16 and
 * lse [rows] fp32; a row with no visible key in any split gets (-inf, 0).
 * MLA_ERR_ARG / MLA_ERR_NULL on bad arguments (host checks), else as
 * mla_verify_attn. */
int mla_verify_lse_combine(int num_splits, int rows,
                           const mla_bf16* part_o,
                           const float* part_lse,
                           mla_bf16* out_latent,
                           float* lse,
                           void* stream);

/* Verify attention with the fused LSE combine + W_UV + sigmoid-gate epilogue
 * (vLLM drafter docstring: "LSE combine + W_UV"; the gate of "gated NoPE
 * MLA" read as an elementwise sigmoid over the 128-d per-head output).
 *   w_uv            [H, 128, 512]  bf16   o_v[d] = sum_c W_UV[h][d][c] o_lat[c]
 *   gate_logits     [B, T, H, 128] bf16
 *   out             [B, T, H, 128] bf16   sigmoid(gate) * o_v
 *   lse             [B, T, H]      fp32
 *   out_latent      [B, T, H, 512] bf16   optional (NULL = not written)
 *   workspace       mla_verify_workspace_size(p, 1) bytes (always > 0)
 * Other arguments and errors as mla_verify_attn. */
int mla_verify_attn_gated(const mla_verify_params* p,
                          const mla_bf16* q_latent,
                          const void* latent_kv_pages,
                          const int32_t* block_table,
                          const int32_t* kv_bounds,
                          const mla_bf16* w_uv,
                          const mla_bf16* gate_logits,
                          mla_bf16* out,
                          float* lse,
                          mla_bf16* out_latent,
                          void* workspace, size_t workspace_bytes,
                          void* stream);

/* mla_verify_attn_gated without a workspace argument, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a static device
 * array of MLA_VERIFY_STATIC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends; the call itself allocates nothing.
 *   Limit: the workspace mla_verify_workspace_size(p, 1) reports must fit the
 *   scratch, else MLA_ERR_WORKSPACE (host check, before any HIP call).
 *   Concurrency: every call on one GPU uses that GPU's one scratch, so calls
 *   that overlap on a GPU (other streams, other threads) race; serialise
 *   them.  Nothing in the scratch needs clearing between calls.
 * Other arguments, results and errors as mla_verify_attn_gated. */
int mla_verify_attn_gated_noalloc(const mla_verify_params* p,
                                  const mla_bf16* q_latent,
                                  const void* latent_kv_pages,
                                  const int32_t* block_table,
                                  const int32_t* kv_bounds,
                                  const mla_bf16* w_uv,
                                  const mla_bf16* gate_logits,
                                  mla_bf16* out,
                                  float* lse,
                                  mla_bf16* out_latent,
                                  void* stream);

/* Query absorption ("absorbed projections", first page, "What does this PR
 * do?"): q_latent[b,t,h,:] = W_UK[h]^T q_nope[b,t,h,:], fp32 accumulation,
 * rounded to bf16 (nearest-even).
 *   q_nope   [B, T, H, 128] bf16,  w_uk [H, 128, 512] bf16,
 *   q_latent [B, T, H, 512] bf16 (output).
 * Uses batch, q_len, num_heads of `p` (other fields are validated as for
 * the attention calls).  No workspace. */
int mla_verify_absorb_q(const mla_verify_params* p,
                        const mla_bf16* q_nope,
                        const mla_bf16* w_uk,
                        mla_bf16* q_latent,
                        void* stream);

/* KV append with a per-token slot table ("Kimi K3: DSpark speculative
 * decoding under Helix CP", first commit message, "Per-token primitive" and
 * "mla_rope_generation", and the same items under "Changes"): every token of
 * a verify group carries its own rank-local KV write slot, -1 when the token
 * is not owned here, and the per-token table supersedes a per-sequence gate.
 * A slot is a request-logical key position (the key the attention calls
 * address as j), so for every (b, t) with 0 <= slots[b,t] < P*64:
 *     latent_kv_pages[block_table[b, slot / 64], slot % 64, :] = new_latent[b, t, :]
 * The latent is written as given (NoPE: no rotary part).  Run it before the
 * attention calls of the same step, whose bounds then cover the new keys.
 *   new_latent       [B, T, 512] bf16   the group's compressed KV
 *   slots            [B, T]      int32  write position, -1 = skip
 *   block_table      [B, P]      int32
 *   latent_kv_pages  [N, 64, 512] bf16  updated in place
 *   bad_slots        int32 counter or NULL: incremented (device atomic) once
 *                    for every token whose slot is below -1 or at least P*64,
 *                    or whose page id lies outside [0, N); such a token writes
 *                    nothing.  The caller zeroes it.
 * Two tokens with the same slot: one of the two rows is written (which one
 * is unspecified).  Shapes: 1 <= B, 1 <= T <= 16, P >= 1, N >= 1 (else
 * MLA_ERR_SHAPE / MLA_ERR_ARG); pointers as for the other calls, bad_slots
 * excepted (4-byte aligned or NULL). */
int mla_verify_kv_append(int batch, int q_len, int max_pages_per_req, int num_pool_pages,
                         const mla_bf16* new_latent,
                         const int32_t* slots,
                         const int32_t* block_table,
                         mla_bf16* latent_kv_pages,
                         int32_t* bad_slots,
                         void* stream);

/* Trim of rejected tails (first page, "What does this PR do?", "Speculative
 * decoding": verification keeps the target token and the accepted drafts, and
 * the KV cache trims the rejected tail).  Request b held kv_len[b] keys after
 * the append, the group's T = k+1 tokens last; it keeps its target token and
 * a = clamp(accepted[b], 0, T-1) drafts, so with L = clamp(kv_len[b], 0, P*64):
 *     new_len[b] = max(0, L - (T - 1 - a))
 * A page that held only dropped keys (page p with new_len <= 64 p < L; since
 * T <= 16 there is at most one) is released: its id is written to
 * released_page[b] and block_table[b, p] is set to -1; released_page[b] = -1
 * when no page is released.
 *   kv_len, accepted  [B] int32;  new_len [B] int32 (may alias kv_len);
 *   block_table [B, P] int32 (updated in place);  released_page [B] int32.
 * Shapes as mla_verify_kv_append. */
int mla_verify_kv_trim(int batch, int q_len, int max_pages_per_req,
                       const int32_t* kv_len,
                       const int32_t* accepted,
                       int32_t* new_len,
                       int32_t* block_table,
                       int32_t* released_page,
                       void* stream);

/* Static, human-readable text for a status code. */
const char* mla_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */
