/*
 * ltxa.h -- C ABI of libltxa.so: masked rotary attention for one
 * sequence-parallel (SP) rank's share, on AMD Instinct MI355X (gfx950).
 *
 * The operations follow two source pages:
 *  - LTX-2 multi-GPU docs, "Sequence Parallelism (SP)": the video sequence is
 *    padded to a multiple of world_size (padded keys masked, padded rows
 *    dropped), Q/K/V are exchanged so that each rank holds every token for a
 *    subset of heads, each rank runs global attention over all tokens for its
 *    heads, and results are shuffled back; the exchange moves bytes only and
 *    num_heads must be divisible by world_size ("What it is", "How the
 *    forward pass works", "API / AttentionManager").
 *  - FastVideo API, fastvideo.models.encoders.gemma: LTXRopeType (INTERLEAVED
 *    pairs 2i, 2i+1), precompute_ltx_freqs_cis (positions normalised by a
 *    per-axis max_pos, base theta) and apply_ltx_rotary_emb.
 *
 * Conventions shared by every call:
 *  - Tensors are caller-owned DEVICE memory, contiguous, row-major.  "BSHD"
 *    means [batch, tokens, heads, head_dim] with head_dim fastest.
 *  - bf16 means IEEE bfloat16 stored as 16-bit words.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it: they never synchronise the host, allocate, free, or
 *    keep a pointer after returning.  Completion follows stream order.
 *  - Every argument is checked before anything is enqueued; on any error the
 *    call returns a negative LTXA_E_* code and enqueues nothing.  The
 *    exception is LTXA_E_HIP, which reports a failed launch.
 *  - The library holds no mutable global state; calls are thread-safe.
 *  - Sizes are 64-bit where they count tokens or elements.
 */
#ifndef LTXA_H
#define LTXA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LTXA_VERSION 107 /* major*100 + minor */

enum ltxa_status {
  LTXA_OK = 0,
  LTXA_E_NULL = -1,         /* a required pointer is NULL */
  LTXA_E_SHAPE = -2,        /* a size is out of range (see each call) */
  LTXA_E_DIVISIBILITY = -3, /* heads or tokens not divisible by world_size */
  LTXA_E_ALIGN = -4,        /* a device pointer is not 16-byte aligned */
  LTXA_E_ALIAS = -5,        /* buffers that must be distinct overlap */
  LTXA_E_HIP = -6,          /* the HIP runtime reported a launch error */
  LTXA_E_RANGE = -7         /* a size overflows 64-bit byte counts or grid limits */
};

/* Library version, LTXA_VERSION of the build. */
int ltxa_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ltxa_status_string(int status);

/*
 * ltxa_sp_pack -- token-major -> per-rank head shards (the one-GPU share of
 * the SP all2all; "What it is" on the SP page).
 *
 *   src: [batch, n_tokens, heads, head_dim] elements of elem_bytes each.
 *   dst: [world_size, batch, n_tokens, heads/world_size, head_dim].
 *   dst[p][b][n][j][:] = src[b][n][p*(heads/world_size) + j][:]
 *
 * Rank p's receive buffer is dst[p], itself a BSHD tensor over all tokens
 * with heads/world_size heads.  A pure byte copy.
 * Errors: E_NULL (src or dst NULL); E_SHAPE (a size < 1, or elem_bytes not in
 * {1,2,4,8}); E_DIVISIBILITY (heads % world_size != 0, or n_tokens %
 * world_size != 0: the SP page pads the sequence to a multiple of
 * world_size first); E_ALIAS (src and dst byte ranges overlap); E_RANGE
 * (a tensor above 2^38 bytes, or world_size above 65535).
 * Any pointer alignment is accepted; 16-byte aligned rows are fastest.
 */
int ltxa_sp_pack(const void* src, void* dst, int64_t batch, int64_t n_tokens,
                 int32_t heads, int32_t head_dim, int32_t world_size,
                 int32_t elem_bytes, void* stream);

/*
 * ltxa_sp_unpack -- inverse of ltxa_sp_pack (results shuffled back to token
 * order; SP page, "What it is").  Same arguments with src and dst roles
 * swapped: src is [world_size, batch, n_tokens, heads/world_size, head_dim],
 * dst is [batch, n_tokens, heads, head_dim].  Same errors.
 */
int ltxa_sp_unpack(const void* src, void* dst, int64_t batch, int64_t n_tokens,
                   int32_t heads, int32_t head_dim, int32_t world_size,
                   int32_t elem_bytes, void* stream);

/*
 * ltxa_rope_qk -- interleaved rotary embedding applied in place to Q and K
 * (FastVideo gemma page: LTXRopeType INTERLEAVED, precompute_ltx_freqs_cis,
 * apply_ltx_rotary_emb).
 *
 *   q: bf16 BSHD [batch, nq, heads, head_dim], rotated in place, may be NULL.
 *   k: bf16 BSHD [batch, nk, heads, head_dim], rotated in place, may be NULL.
 *   q_pos / k_pos: DEVICE int32 [nq, q_axes] / [nk, k_axes] integer
 *     positions (axis order t, x, y for 3 axes; time for 1 axis), shared by
 *     every batch entry and head.
 *   q_max_pos / k_max_pos: HOST arrays of q_axes / k_axes positive values,
 *     read during the call only.
 *   theta: frequency base (the pages' default is 10000).
 *
 * With A axes and head_dim/2 channel pairs, axis a owns the n_ax =
 * floor(head_dim/2/A) consecutive pairs starting at a*n_ax; pair a*n_ax + k
 * turns by phi = (pos[a] / max_pos[a]) * theta^(-k/n_ax); the
 * (head_dim/2) mod A highest pairs are left as they are.  Pair (x0, x1) =
 * channels (2i, 2i+1) becomes (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos
 * phi).  Angles and products are computed in fp32 from fp64 per-pair
 * frequencies; results are rounded to bf16 (nearest even).  When q and k
 * are both given with the same q_pos pointer, token count, axis count and
 * max_pos values (self-attention), one kernel rotates both and computes each
 * angle once; the bits are those of two separate calls.
 * Errors: E_NULL (both q and k NULL, or a non-NULL tensor without its
 * positions or max_pos); E_SHAPE (batch, heads or a token count < 1, head_dim
 * odd or not in [2, 256], axes not in {1,2,3} or more axes than pairs,
 * max_pos <= 0 or not finite, theta <= 0 or not finite); E_ALIGN (q, k or a
 * position array not 16-byte aligned, or head_dim*2 not a multiple of 16);
 * E_ALIAS (q and k overlap); E_RANGE.
 */
int ltxa_rope_qk(void* q, const int32_t* q_pos, int64_t nq, int32_t q_axes,
                 const double* q_max_pos,
                 void* k, const int32_t* k_pos, int64_t nk, int32_t k_axes,
                 const double* k_max_pos,
                 int64_t batch, int32_t heads, int32_t head_dim, double theta,
                 void* stream);

/*
 * ltxa_attn_fwd -- key-padding-masked scaled-dot-product attention over all
 * tokens for the given heads (SP page, "What it is": attention stays global;
 * "How the forward pass works" step 1: padded keys are masked out).
 *
 *   q: bf16 BSHD [batch, nq, heads, head_dim]
 *   k, v: bf16 BSHD [batch, nk_pad, heads, head_dim]
 *   o: bf16 BSHD [batch, nq, heads, head_dim] (written)
 *   lse: fp32 [batch, heads, nq] natural-log log-sum-exp of the scaled
 *     scores per query row, or NULL.
 *   For each b, h and query i: s_ij = scale * <q_i, k_j> over keys
 *   j < nk_valid only; o_i = sum_j softmax_j(s_i) v_j.  Keys at or past
 *   nk_valid are never read, so their contents (NaN included) cannot reach
 *   the output.  Query rows past the caller's valid length are computed like
 *   any other row.
 * Arithmetic: q is multiplied by c = scale * log2(e) (both in fp32) and
 * rounded to bf16 once: each element moves by at most 2^-8 of its value
 * (bf16 keeps 8 significant bits), so the natural-log score s_ij moves by at
 * most 2^-8 * scale * sum_d |q_id k_jd|.  Then exact bf16 products with fp32
 * accumulation, a base-2 softmax in fp32 whose probabilities are rounded to
 * bf16 (at most 2^-8 relative) for the weighted sum of v and summed
 * unrounded in fp32 for the row sum, and fp32 -> bf16 output rounding
 * (nearest even).  So, with
 * delta_i = 2^-8 * scale * max_j sum_d |q_id k_jd| - ln(1 - 2^-8) plus
 * fp32 accumulation terms: |lse_i - exact| <= delta_i, and every softmax
 * weight is within a factor e^(+-2 delta_i) of the exact one.
 * Inputs: Q and the K/V rows below nk_valid are expected to be finite.  A NaN
 * or infinity there is not hidden: it makes non-finite every output row it
 * reaches (its own row for a Q value; every row of the head for a K or V
 * value).  The other rows keep the accuracy stated above; other heads are
 * not affected at all.
 * Errors: E_NULL (q, k, v or o NULL); E_SHAPE (batch, heads, nq < 1;
 * head_dim not 64 or 128; nk_valid not in [1, nk_pad]; scale not finite and
 * > 0); E_ALIGN (a pointer not 16-byte aligned); E_ALIAS (o or lse overlaps
 * q, k, v, or each other); E_RANGE.
 */
int ltxa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                  int64_t nk_pad, int64_t nk_valid, float scale, void* stream);

/*
 * ltxa_sp_pack_rope -- ltxa_sp_pack and the rotary embedding of
 * ltxa_rope_qk in one pass over memory (the SP page's exchange of Q or K,
 * "What it is", followed by the FastVideo gemma page's
 * apply_ltx_rotary_emb; the rotation acts per token and per pair, so it
 * commutes with the head permutation).
 *
 *   src: bf16 [batch, n_tokens, heads, head_dim], read only.
 *   dst: bf16 [world_size, batch, n_tokens, heads/world_size, head_dim]:
 *     dst[p][b][n][j] = rotate(src[b][n][p*(heads/world_size) + j], pos[n]).
 *   pos: DEVICE int32 [n_tokens, axes]; max_pos: HOST array of `axes`
 *     values; theta: frequency base.  The angle schedule, the arithmetic and
 *     the rounding are those of ltxa_rope_qk, so dst equals, bit for bit,
 *     ltxa_sp_pack followed by ltxa_rope_qk on the packed tensor (positions
 *     shared by every rank).
 * Errors: E_NULL (src, dst, pos or max_pos NULL); E_SHAPE (as ltxa_rope_qk
 * for sizes, axes, max_pos and theta; world_size < 1); E_DIVISIBILITY (as
 * ltxa_sp_pack); E_ALIGN (src, dst or pos not 16-byte aligned, or
 * head_dim*2 not a multiple of 16); E_ALIAS (src and dst overlap); E_RANGE.
 */
int ltxa_sp_pack_rope(const void* src, void* dst, const int32_t* pos, int64_t n_tokens,
                      int32_t axes, const double* max_pos, int64_t batch, int32_t heads,
                      int32_t head_dim, int32_t world_size, double theta, void* stream);

/*
 * ltxa_attn_fwd_unpack -- ltxa_attn_fwd on every rank's head shard with the
 * output written straight into token order (SP page, "What it is": each rank
 * attends over all tokens for its heads, then results are shuffled back).
 *
 *   q: bf16 [world_size, batch, nq, heads/world_size, head_dim]
 *   k, v: bf16 [world_size, batch, nk_pad, heads/world_size, head_dim]
 *     (the layout ltxa_sp_pack / ltxa_sp_pack_rope write).
 *   o: bf16 [batch, nq, heads, head_dim] (written): rank p's head j lands at
 *     head p*(heads/world_size) + j.
 *   lse: fp32 [world_size, batch, heads/world_size, nq], or NULL.
 *   batch and heads are the unsharded counts.  Masking, scale and
 *   arithmetic are those of ltxa_attn_fwd; o equals, bit for bit,
 *   ltxa_attn_fwd over the world_size * batch shard entries followed by
 *   ltxa_sp_unpack.
 * Errors: those of ltxa_attn_fwd for world_size * batch entries of
 * heads/world_size heads; E_SHAPE (world_size < 1); E_DIVISIBILITY
 * (heads % world_size != 0).
 */
int ltxa_attn_fwd_unpack(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                         int64_t nk_pad, int64_t nk_valid, float scale, int32_t world_size,
                         void* stream);

/*
 * Rotary variants (FastVideo gemma page: LTXRopeType's two pairings;
 * precompute_ltx_freqs_cis's grid width `dim` with `num_attention_heads`,
 * its `use_middle_indices_grid`, and the float64 grid generator that
 * double_precision_rope selects).
 */
#define LTXA_ROPE_INTERLEAVED 0 /* pairs (2i, 2i+1) */
#define LTXA_ROPE_SPLIT 1       /* pairs (i, i + head_dim/2) */

typedef struct ltxa_rope_opts {
  int32_t rope_type;   /* LTXA_ROPE_INTERLEAVED or LTXA_ROPE_SPLIT */
  int32_t grid_heads;  /* 0: one grid over head_dim shared by every head.
                          G >= 1: one grid over G * head_dim channels
                          (G * head_dim / 2 pairs, n_ax = floor(that / axes)
                          per axis); grid head g turns its pairs by the
                          global pairs [g*head_dim/2, (g+1)*head_dim/2) */
  int32_t head_offset; /* with grid_heads > 0: grid head of the tensor's head 0 */
  int32_t fp64_angles; /* 0: angle and sin/cos in fp32; 1: in fp64 (the
                          rotation itself stays fp32) */
  int32_t middle;      /* 0: angle uses pos; 1: pos + 1/2 (cell middles) */
  float out_scale;     /* 0: none.  Otherwise finite and > 0: every output
                          value is the rotated value times out_scale,
                          rounded to bf16 once (cos and sin are multiplied
                          by it in fp32, once per token and pair; channels
                          the rotation leaves alone are scaled too).  With
                          out_scale = scale * log2(e) the result is the q
                          operand of the _log2q attention calls below. */
} ltxa_rope_opts;

/*
 * ltxa_rope_ex -- rotary embedding of one bf16 tensor in place with the
 * variants above (opts NULL = all zero = the rotation of ltxa_rope_qk,
 * bit for bit).
 *
 *   x: bf16 [batch, n_tokens, heads, head_dim], rotated in place.
 *   pos: DEVICE int32 [n_tokens, axes]; max_pos: HOST array of `axes`
 *     values; theta: frequency base.
 *   With grid_heads = G > 0, head j of x is grid head head_offset + j, so
 *   head_offset + heads <= G.  A buffer of several ranks' head shards is
 *   rotated one rank at a time (head_offset = rank * heads per rank), or
 *   through ltxa_sp_pack_rope_ex.
 * Errors: as ltxa_rope_qk for one tensor, plus E_NULL (pos or max_pos NULL),
 * E_SHAPE (rope_type, fp64_angles or middle not 0/1; out_scale neither 0
 * nor finite and > 0; grid_heads < 0, head_offset < 0 or head_offset +
 * heads > grid_heads; fewer grid pairs than axes), E_ALIGN (SPLIT with
 * head_dim % 16 != 0).
 */
int ltxa_rope_ex(void* x, const int32_t* pos, int64_t n_tokens, int32_t axes,
                 const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim,
                 double theta, const ltxa_rope_opts* opts, void* stream);

/*
 * ltxa_rope_qk_ex -- ltxa_rope_ex of Q and of K in one launch, for a layer
 * whose queries and keys turn by the same positions and options (the text
 * connector's self-attention on the FastVideo gemma page: one 1D position
 * grid, laid over the inner dimension of all heads, applied to Q and K).
 * Each angle is evaluated once for both tensors.
 *   q, k: bf16 [batch, n_tokens, heads, head_dim], rotated in place; they
 *     may not overlap.
 *   opts: as for ltxa_rope_ex; its out_scale applies to q only.
 *   k_scale: 0 (none), or finite and > 0: every rotated value of k is
 *     multiplied by it before its one rounding.
 * q and k equal, bit for bit, ltxa_rope_ex(q, ..., opts) and
 * ltxa_rope_ex(k, ..., opts with out_scale = k_scale).
 * Errors: those of ltxa_rope_ex for q; E_NULL (k NULL); E_SHAPE (k_scale
 * neither 0 nor finite and > 0); E_ALIGN (k not 16-byte aligned); E_ALIAS
 * (k overlaps q or pos).
 */
int ltxa_rope_qk_ex(void* q, void* k, const int32_t* pos, int64_t n_tokens, int32_t axes,
                    const double* max_pos, int64_t batch, int32_t heads, int32_t head_dim,
                    double theta, const ltxa_rope_opts* opts, float k_scale, void* stream);

/*
 * ltxa_sp_pack_rope_ex -- ltxa_sp_pack_rope with the variants above: the
 * source head h (of `heads`) is grid head head_offset + h.  dst equals, bit
 * for bit, ltxa_sp_pack followed by ltxa_rope_ex on each rank's shard with
 * that rank's head offset.  Errors: those of ltxa_sp_pack_rope and
 * ltxa_rope_ex.
 */
int ltxa_sp_pack_rope_ex(const void* src, void* dst, const int32_t* pos, int64_t n_tokens,
                         int32_t axes, const double* max_pos, int64_t batch, int32_t heads,
                         int32_t head_dim, int32_t world_size, double theta,
                         const ltxa_rope_opts* opts, void* stream);

/*
 * Angle tables.  The FastVideo gemma page computes the rotary frequencies
 * once (precompute_ltx_freqs_cis) and applies them to each tensor later
 * (apply_ltx_rotary_emb).  The two calls below split the head-shared grid
 * the same way: the angles of a position buffer are evaluated once into a
 * caller-owned table, and every tensor rotated with those positions reads
 * them.
 *
 * ltxa_rope_table -- cos and sin of every (token, pair) of the head-shared
 * grid.
 *   pos: DEVICE int32 [n_tokens, axes]; max_pos: HOST array of `axes`
 *     values; theta: frequency base; head_dim: channels per head.
 *   opts: NULL or the variants above; only fp64_angles and middle act.
 *     rope_type does not change a pair's angle.  grid_heads and out_scale
 *     must be 0: the table serves the head-shared grid, and scaling belongs
 *     to the rotation.
 *   table: DEVICE fp32 [n_tokens, head_dim/2, 2] (written, caller-owned):
 *     table[n][i] = (cos, sin) of pair i's angle for token n, evaluated
 *     exactly as ltxa_rope_ex evaluates it (1 and 0 for the pairs the
 *     schedule leaves unrotated).
 * Errors: E_NULL (pos, max_pos or table NULL); E_SHAPE (as ltxa_rope_ex for
 * head_dim, axes, max_pos, theta and opts; grid_heads or out_scale not 0);
 * E_ALIGN (pos or table not 16-byte aligned, or head_dim*2 not a multiple
 * of 16); E_ALIAS (table overlaps pos); E_RANGE.
 */
int ltxa_rope_table(const int32_t* pos, int64_t n_tokens, int32_t axes, const double* max_pos,
                    int32_t head_dim, double theta, const ltxa_rope_opts* opts, float* table,
                    void* stream);

/*
 * ltxa_sp_pack_rope_table -- ltxa_sp_pack_rope_ex with the angles read from
 * a table of ltxa_rope_table.
 *   src: bf16 [batch, n_tokens, heads, head_dim], read only.
 *   dst: bf16 [world_size, batch, n_tokens, heads/world_size, head_dim],
 *     written.
 *   table: DEVICE fp32 [n_tokens, head_dim/2, 2], read only.
 *   rope_type: LTXA_ROPE_INTERLEAVED or LTXA_ROPE_SPLIT.
 *   out_scale: 0 (none), or finite and > 0, as in ltxa_rope_opts.
 * dst equals, bit for bit, ltxa_sp_pack_rope_ex with the opts the table was
 * made with, plus this rope_type and out_scale.
 * Errors: E_NULL (src, dst or table NULL); E_SHAPE (a size < 1, head_dim
 * odd or above 256, rope_type not 0/1, out_scale neither 0 nor finite and
 * > 0); E_DIVISIBILITY (as ltxa_sp_pack); E_ALIGN (src, dst or table not
 * 16-byte aligned, head_dim*2 not a multiple of 16, or SPLIT with
 * head_dim % 16 != 0); E_ALIAS (dst overlaps src or table); E_RANGE.
 */
int ltxa_sp_pack_rope_table(const void* src, void* dst, const float* table, int64_t n_tokens,
                            int64_t batch, int32_t heads, int32_t head_dim, int32_t world_size,
                            int32_t rope_type, float out_scale, void* stream);

/*
 * ltxa_sp_pack_rope_qk_table -- ltxa_sp_pack_rope_table of Q and of K in one
 * launch, for self-attention, where Q and K of a token turn by the same
 * angles (the rotary embedding page's precomputed frequencies, applied to
 * the queries and the keys alike).  Each table entry is read once for both.
 *   q, k: bf16 [batch, n_tokens, heads, head_dim], read only (they may
 *     overlap each other).
 *   q_dst, k_dst: bf16 [world_size, batch, n_tokens, heads/world_size,
 *     head_dim], written.
 *   q_scale, k_scale: the out_scale of each (0 = none).
 *   table, rope_type and the sizes: as in ltxa_sp_pack_rope_table.
 * q_dst and k_dst equal, bit for bit, ltxa_sp_pack_rope_table(q, q_dst, ...,
 * q_scale) and ltxa_sp_pack_rope_table(k, k_dst, ..., k_scale).
 * Errors: those of ltxa_sp_pack_rope_table for either pair, and E_ALIAS when
 * q_dst overlaps k or k_dst, or k_dst overlaps q.
 */
int ltxa_sp_pack_rope_qk_table(const void* q, void* q_dst, float q_scale, const void* k, void* k_dst,
                               float k_scale, const float* table, int64_t n_tokens, int64_t batch,
                               int32_t heads, int32_t head_dim, int32_t world_size, int32_t rope_type,
                               void* stream);

/*
 * Log2-domain queries.  The attention computes its softmax in base 2: with
 * c = scale * log2(e), exp(scale * <q, k>) = 2^<c q, k>.  ltxa_attn_fwd
 * multiplies q by c itself and rounds the product to bf16, on top of the
 * rounding that produced q (the rotary embedding's, in the SP page's
 * exchange of Q).  The rotary calls with opts->out_scale = c make that
 * product ahead of their one rounding, and the two calls below take such q
 * as given, so that each q value is rounded once in all.
 */

/*
 * ltxa_attn_fwd_log2q -- ltxa_attn_fwd for queries already in the log2
 * domain (SP page, "What it is": attention stays global over all tokens).
 * q holds c * q_i for c = scale * log2(e), rounded to bf16 (as
 * ltxa_rope_ex / ltxa_sp_pack_rope_ex with opts->out_scale = c write it),
 * and is used as given: the scores are s_ij = ln(2) * <q_i, k_j>.  Layouts,
 * masking, lse (natural log of the scores) and the rest of the arithmetic
 * are those of ltxa_attn_fwd.  The kernel neither multiplies nor rounds q
 * again, so in ltxa_attn_fwd's bound the 2^-8 * scale * sum_d |q_id k_jd|
 * term stands for the rounding of c * q itself: it is counted once, where
 * ltxa_attn_fwd on a rounded q counts it twice.  With q = bf16(q' * c)
 * formed in fp32, c being the double product scale * log2(e) rounded to
 * fp32 (what ltxa_attn_fwd uses), o and lse equal ltxa_attn_fwd(q', scale)
 * bit for bit.
 * Errors: those of ltxa_attn_fwd (there is no scale to check).
 */
int ltxa_attn_fwd_log2q(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                        int64_t nk_pad, int64_t nk_valid, void* stream);

/*
 * ltxa_attn_fwd_unpack_log2q -- ltxa_attn_fwd_unpack for log2-domain
 * queries: the q operand, arithmetic and bit-exactness statement of
 * ltxa_attn_fwd_log2q, the layouts of ltxa_attn_fwd_unpack (q as
 * ltxa_sp_pack_rope_ex with opts->out_scale = c writes it).  o and lse equal
 * ltxa_attn_fwd_log2q over the world_size * batch shard entries followed by
 * ltxa_sp_unpack, bit for bit.
 * Errors: those of ltxa_attn_fwd_unpack (there is no scale to check).
 */
int ltxa_attn_fwd_unpack_log2q(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t batch, int32_t heads, int32_t head_dim, int64_t nq,
                               int64_t nk_pad, int64_t nk_valid, int32_t world_size, void* stream);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* LTXA_H */
