/*
 * akv.h -- split-KV, two-tier decode attention for AMD Instinct MI355X (gfx950).
 *
 * A key/value history is held in two tiers, after the two-precision cache of
 * ActiveKV ("Context beyond VRAM", section "What I built"): a window of the
 * newest tokens in full precision, the older tokens in a small encoded form
 * that the attention kernels read in place, and one exact log-sum-exp merge
 * joining the two:
 *
 *   exact tier       bfloat16 K and V, paged in 64-token blocks;
 *   compressed tier  K and V rotated by the normalized Walsh-Hadamard matrix
 *                    H_d/sqrt(d), cut into 32-element groups, each group stored
 *                    as one fp16 RMS scale plus 4-bit indices into the 16-level
 *                    Lloyd-Max table for N(0,1).  Because the rotation keeps dot
 *                    products, the query is rotated once instead of inverse-
 *                    rotating the blocks (QuantForge walkthrough, section 1,
 *                    "Triton Fused Kernels").
 *
 * Each tier is attended in fixed-size token splits; every split yields a
 * normalized partial output and its log-sum-exp (the attention statistic that
 * "Bringing a serving stack up on new silicon", section "What I built", adds to
 * the paged-attention path), and the partials are combined by an exact
 * log-sum-exp merge in a fixed order, so repeated calls are bit-identical.
 *
 * Conventions for every entry point (the port described in "PyTorch",
 * section "Native operators inside vLLM", kept shapes, dtypes, lifetimes, the
 * caller's device stream and the order of error reports):
 *   - all tensor pointers are DEVICE pointers unless stated; the caller owns
 *     every buffer (including the workspace) and keeps it alive until the work
 *     enqueued on `stream` has finished;
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream);
 *     the library only enqueues work on it, never synchronizes, never
 *     allocates or frees device memory, and keeps no pointer after returning;
 *   - arguments are validated on the host before anything is enqueued, in the
 *     fixed order NULL -> SHAPE -> UNSUPPORTED -> ALIGN -> WORKSPACE; the first
 *     failure is returned and nothing has been enqueued.  A request that cannot
 *     be served is refused, never truncated (ActiveKV, "What I built":
 *     unservable requests are refused);
 *   - a HIP launch failure returns AKV_ERR_HIP; akv_last_error() then holds
 *     the HIP error string.  akv_last_error() is thread-local.
 *   - device-side data errors that the host cannot see (a block-table entry
 *     outside [0, num_blocks), a length above 64*max_blocks) make the affected
 *     (sequence, head) outputs NaN instead of faulting.
 *
 * ---------------------------------------------------------------- layouts
 * Hkv = key/value heads, d = head dimension (64 or 128), G = Hq/Hkv <= 8;
 * query head h reads key/value head h / G.  A block holds 64 tokens.
 *
 * Exact tier pools: bf16, element (block p, kv head k, token r, dim t) at
 *   K: ((p*Hkv + k)*64 + r)*d + t                   (token-major)
 *   V: (((p*Hkv + k)*2 + r/32)*d + t)*32 + r%32     (dim-major inside each
 *                                                    32-token half block)
 * so that a lane's matrix-core operand (8 dims of one token for K, 8 tokens
 * of one dim for V) is one contiguous 16-byte load, and the 64 lanes of one
 * load instruction read 1 KB of consecutive bytes.  Appending a token writes
 * one row of K and one bf16 per dim of V.
 *
 * Compressed tier: one slab of 32*d code bytes and one slab of 2*d fp16
 * scales per (block p, kv head k), at byte offset (p*Hkv + k)*32*d and element
 * offset (p*Hkv + k)*2*d.  Codes are 4-bit values 0..15; byte = lo | hi << 4.
 *   K codes: token r owns bytes [r*d/2, (r+1)*d/2); inside that row, byte
 *     (d/8)*a + 4*m + b  (a = 0..3, m = 0..d/32-1, b = 0..3) holds dims
 *     32m + 8a + 2b (low nibble) and 32m + 8a + 2b + 1 (high nibble).
 *   V codes: byte c*16*d + (t/4)*1024 + (a*16 + i)*16 + 4*(t%4) + b
 *     (c = 0..1, a = 0..3, i = 0..15, t = 0..d/16-1, b = 0..3) holds dim
 *     16t + i of tokens 32c + 8a + 2b (low nibble) and 32c + 8a + 2b + 1
 *     (high nibble).
 *   K and V scales: fp16, element g*64 + r = group g (dims 32g..32g+31) of
 *     token r.
 * These orders put each lane's matrix-core operand in one contiguous load.
 * Dequantized (rotated-space) value of dim t of a token: C[code] * scale(t/32),
 * with C the Lloyd-Max table; the unrotated vector is (H_d/sqrt(d)) times it.
 *
 * Rotation (the QuantForge walkthrough, section 5, sets the Hadamard rotation
 * against a QR, i.e. random orthogonal, one): every descriptor that encodes
 * or reads the compressed tier has a `rotation` field.  NULL selects the
 * normalized Walsh-Hadamard rotation above.  Otherwise it is a device
 * pointer to a float32 [d][d] row-major orthogonal matrix R, 16-byte
 * aligned: the encoder stores codes of y = R x (y_i summed in ascending k,
 * one float32 multiply and add per term, no 1/sqrt(d) step), decode and the
 * prefill chunk rotate each query by R once per call (workspace grows by
 * 4*B*Tq*Hq*d bytes) and the compressed-tier output by R^T once per
 * (query, head), and the unrotated vector is R^T times the rotated one.  The
 * same R must be used to encode and to attend.
 *
 * Code width: every descriptor that encodes or reads the compressed tier has
 * a `code_bits` field, w = 4 (or 0) for the 16-level table and layout above,
 * 2 or 3 for the 4- or 8-level Lloyd-Max table for N(0,1); only the table and
 * the code bytes change, scales and every other step do not (an all-zero
 * group gets code 2^(w-1) - 1).  A width-w code slab has 8*w*d bytes per
 * (block p, kv head k), at byte offset (p*Hkv + k)*8*w*d.
 *   w = 2: a pair plane.  A 4-bit field holds two codes (first | second << 2)
 *     and a byte two fields (bits 0..3 and 4..7, h = 0 and 1):
 *     K: token r owns bytes [r*d/4, (r+1)*d/4); byte (d/16)*a + 4*n + b holds
 *       in field h dims 32(2n + h) + 8a + 2b and + 1;
 *     V: byte ((c*4 + a)*16 + i)*(d/8) + 4*n + b holds in field h dim
 *       16(2n + h) + i of tokens 32c + 8a + 2b and + 1.
 *   w = 3: the pair plane of the codes' low two bits (16*d bytes), then a high
 *     plane of their top bits (8*d bytes) where a 2-bit field holds the top
 *     bits of two codes (first | second << 1):
 *     K: token r owns bytes [r*d/8, (r+1)*d/8) of the high plane; with
 *       M = d/32, row bits 8*M*a + 2*M*b + 2*m + {0, 1} hold dims
 *       32m + 8a + 2b and + 1;
 *     V: byte ((c*4 + a)*16 + i)*(d/16) + 4*n + b, bits 2*h + {0, 1}, holds
 *       dim 16(4n + h) + i of tokens 32c + 8a + 2b and + 1.
 *
 * Block tables: int32 [B][max_blocks]; entry j of row b is the pool block of
 * tier-local tokens [64j, 64j+64) of sequence b.  Tier lengths: int32 [B].
 * In the attended history of a sequence the compressed tier comes first
 * (older), then the exact tier.
 */
#ifndef AKV_H
#define AKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AKV_ABI_VERSION 1
#define AKV_BLOCK_TOKENS 64
#define AKV_GROUP 32
/* Fixed split rule (the lengths never enter it, so repeated calls on one
 * shape partition the history identically): a tier of n tokens is cut into
 * ceil(n / P) splits of P tokens, the last one shorter.  A descriptor may pass
 * P (a multiple of 64) per tier; 0 picks the default from the shape alone.
 * akv_attend_decode's default aims at one round of workgroups: with
 * budget = AKV_DECODE_TARGET_WORKGROUPS / (B * Hkv) splits per kv head and
 * tier capacities Nq = 64 * quant.max_blocks, Ne = 64 * exact.max_blocks
 * tokens, the compressed tier takes the smallest Pq in 256, 512, 768 with
 * ceil(Nq / Pq) + ceil(Ne / AKV_SPLIT_TOKENS_EXACT_DEFAULT) <= budget; when
 * none fits (no single round), Pq = ceil(Nq * B * Hkv /
 * AKV_DECODE_MANY_WORKGROUPS) rounded up to a multiple of 256, at least
 * AKV_SPLIT_TOKENS_QUANT_DEFAULT and at most AKV_MAX_SPLIT_TOKENS (a few
 * rounds of longer workgroups).  With rem = budget - ceil(Nq / Pq) >= 1 the
 * exact tier takes Pe = 64 * ceil(exact.max_blocks / rem) clamped to
 * [AKV_MIN_SPLIT_TOKENS, AKV_SPLIT_TOKENS_EXACT_DEFAULT], else the default.
 * E.g. 1 sequence, 4 kv heads, 123,904 + 4,096 tokens: Pq = 1024 (121
 * splits), Pe = 640 (7 splits), 512 workgroups; 32 sequences on 4 kv heads
 * with tables of 880 compressed + 32 exact blocks: Pq = 3584 (16 splits),
 * Pe = 1024 (2 splits). */
#define AKV_SPLIT_TOKENS_EXACT_DEFAULT 1024
#define AKV_SPLIT_TOKENS_QUANT_DEFAULT 1024
#define AKV_MIN_SPLIT_TOKENS 256
#define AKV_DECODE_TARGET_WORKGROUPS 512   /* two per compute unit on 256 CUs */
#define AKV_DECODE_MANY_WORKGROUPS 2048    /* about four rounds */
/* A decode grid whose splits give fewer workgroups than compute units attends
 * every split with `sub` workgroups (equal runs of whole blocks, each at least
 * AKV_MIN_SUBSPLIT_BLOCKS blocks; sub the largest of AKV_DECODE_MAX_SUBSPLITS,
 * ..., 4, 2 with B * Hkv * splits * sub <= AKV_DECODE_TARGET_WORKGROUPS / 2
 * that divides every present tier's split blocks by AKV_MIN_SUBSPLIT_BLOCKS
 * runs), because one compute unit streams only part of what HBM delivers.
 * Their partials are merged in ascending token order inside the call, so a
 * split stays the unit of the caller's partition; the choice depends on the
 * shape only.  E.g. 32,768 exact tokens in 16 splits of 2,048 on 4 kv heads:
 * 4 workgroups of 512 tokens per split. */
#define AKV_DECODE_MAX_SUBSPLITS 8
#define AKV_MIN_SUBSPLIT_BLOCKS 4
/* akv_attend_chunk's default instead: with Tq*G rows per kv head taken in
 * row groups of AKV_CHUNK_ROWS, a tier of max_blocks blocks is cut into
 * want = ceil(AKV_CHUNK_TARGET_WORKGROUPS / (B * Hkv * row groups)) runs of
 * P = 64 * ceil(max_blocks / want) tokens (at most AKV_MAX_SPLIT_TOKENS). */
#define AKV_CHUNK_ROWS 128
#define AKV_CHUNK_TARGET_WORKGROUPS 512
#define AKV_MAX_SPLIT_TOKENS 32768   /* largest split size served */
#define AKV_MAX_SPLITS 2048          /* largest (compressed + exact) splits per sequence */
#define AKV_MAX_CHUNK 512
/* Also AKV_ERR_UNSUPPORTED: B or Hkv above 65535, Tq * Hq above 2^30, and any
 * shape whose partials (B * Hkv * splits * Tq * G rows of d + 1 floats) would
 * need more than 2^50 workspace bytes. */

typedef enum akv_status {
  AKV_OK = 0,
  AKV_ERR_NULL = -1,        /* a required pointer is NULL */
  AKV_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  AKV_ERR_UNSUPPORTED = -3, /* a valid request this library does not serve */
  AKV_ERR_ALIGN = -5,       /* a pointer is not aligned as required */
  AKV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
  AKV_ERR_HIP = -6          /* HIP reported an error while enqueuing */
} akv_status;

/* Exact (bf16) tier of a batch.  Absent when max_blocks == 0 (then the
 * pointers may be NULL and every sequence has 0 exact tokens). */
typedef struct akv_exact_tier {
  const uint16_t* k;           /* bf16 pool, token-major (layout above) */
  const uint16_t* v;           /* bf16 pool, dim-major inside each half block */
  const int32_t* block_table;  /* [B][max_blocks] */
  const int32_t* lengths;      /* [B], 0 <= len <= 64*max_blocks */
  int32_t max_blocks;          /* row stride of block_table */
  int32_t num_blocks;          /* blocks in each pool */
} akv_exact_tier;

/* Compressed tier of a batch (code width: akv_attn_desc.code_bits).  Absent
 * when max_blocks == 0. */
typedef struct akv_quant_tier {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scales;    /* fp16 */
  const uint16_t* v_scales;    /* fp16 */
  const int32_t* block_table;  /* [B][max_blocks] */
  const int32_t* lengths;      /* [B] */
  int32_t max_blocks;
  int32_t num_blocks;
} akv_quant_tier;

/* One attention call over a batch.  For akv_attend_decode Tq must be 1.
 * For akv_attend_chunk Tq = T (1..512) causal queries: the caller has already
 * appended the chunk's own K/V as the last T exact-tier tokens, and query i
 * (0-based) of a sequence sees the whole compressed tier, the exact tier up
 * to and including exact token len_exact - T + i. */
typedef struct akv_attn_desc {
  uint32_t struct_size;        /* sizeof(akv_attn_desc) */
  int32_t B, Hq, Hkv, d, Tq;
  float softmax_scale;         /* 0 => 1/sqrt(d) */
  const uint16_t* q;           /* bf16 [B][Tq][Hq][d], 4-byte aligned */
  akv_exact_tier exact;
  akv_quant_tier quant;
  int32_t split_tokens_exact;  /* 0 => the shape-only default above */
  int32_t split_tokens_quant;  /* 0 => the shape-only default above */
  float* o;                    /* fp32 [B][Tq][Hq][d] normalized output */
  float* lse;                  /* fp32 [B][Tq][Hq] natural-log sum of exp(scores) */
  const float* rotation;       /* NULL, or the compressed tier's rotation R (see "Rotation") */
  int32_t code_bits;           /* compressed-tier code width: 0 or 4, 3, 2 (see "Code width") */
} akv_attn_desc;

typedef akv_attn_desc akv_decode_desc;
typedef akv_attn_desc akv_chunk_desc;

/* Move n_tokens tokens of one sequence from the exact tier into the
 * compressed tier (ActiveKV's compact older history; encoding per the
 * Walsh-Hadamard rotation of the QuantForge walkthrough, section 1).  For each
 * token, kv head and K|V the bf16 vector is rotated by the unnormalized
 * Walsh-Hadamard butterflies in fp32, scaled by RN(1/sqrt(d)), each 32-group
 * gets scale = fp16(sqrt(mean of squares)) and every element the index of
 * the nearest Lloyd-Max level to value/scale (exact ties to the lower index;
 * all-zero groups give index 7, or 2^(w-1) - 1 at code width w).  Codes and
 * scales are bit-exact functions of the input.  Source tokens [src_start,
 * src_start + n_tokens) of the exact tier's block table land at compressed
 * positions [dst_start, dst_start + n_tokens); dst_start may be odd.  Two
 * tokens share each value-code byte, so where the range begins or ends inside
 * such a byte, the half of the neighbouring position is read and kept: no
 * byte outside the range changes.  Each byte has one writer within a call,
 * and calls that write the same compressed positions must not overlap. */
typedef struct akv_compress_desc {
  uint32_t struct_size;        /* sizeof(akv_compress_desc) */
  int32_t Hkv, d;
  const uint16_t* src_k;       /* bf16 exact-tier pools (layouts above) */
  const uint16_t* src_v;
  const int32_t* src_block_table;  /* [src_max_blocks] one sequence's row */
  int32_t src_max_blocks, src_num_blocks;
  int32_t src_start, n_tokens;
  uint8_t* dst_k_codes;
  uint8_t* dst_v_codes;
  uint16_t* dst_k_scales;
  uint16_t* dst_v_scales;
  const int32_t* dst_block_table;  /* [dst_max_blocks] */
  int32_t dst_max_blocks, dst_num_blocks;
  int32_t dst_start;
  const float* rotation;       /* NULL, or the rotation R (see "Rotation") */
  int32_t code_bits;           /* 0 or 4, 3, 2 (see "Code width") */
} akv_compress_desc;

/* ABI version of the loaded library (AKV_ABI_VERSION at build time). */
int akv_abi_version(void);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* akv_last_error(void);

/* Bytes of workspace akv_attend_decode / akv_attend_chunk need for `desc`
 * (per-split partial outputs and statistics).  Returns 0 if desc is invalid. */
size_t akv_decode_workspace_bytes(const akv_attn_desc* desc);
size_t akv_chunk_workspace_bytes(const akv_attn_desc* desc);

/* The split plan a call with `desc` would use (chunk != 0: akv_attend_chunk,
 * else akv_attend_decode): out[0..3] = compressed-tier split tokens, exact-
 * tier split tokens, compressed-tier splits, exact-tier splits per sequence
 * and kv head.  Validates desc like the call itself and returns its status;
 * out (host memory, 4 int32) is written only on AKV_OK. */
akv_status akv_split_plan(const akv_attn_desc* desc, int32_t chunk, int32_t* out);

/* Workgroups that attend each split of an akv_attend_decode call with `desc`
 * (1, or the sub-split count of AKV_DECODE_MAX_SUBSPLITS above); 0 if desc is
 * invalid. */
int32_t akv_decode_split_workgroups(const akv_attn_desc* desc);

/* One sequence's compressed tier held in pinned host memory (hipHostMalloc):
 * ceil(length / 64) block records in token order (record i holds tokens
 * [64i, 64i + 64)), each (16w + 8)*Hkv*d bytes for code width w (72*Hkv*d
 * at w = 4): Hkv K-code slabs (8*w*d bytes each), Hkv V-code slabs, Hkv
 * K-scale slabs (2*d fp16 each), Hkv V-scale slabs,
 * with the per-slab layouts above.  This is the record layout of a
 * checkpoint image's compressed slots, so a sequence's slots of an image in
 * pinned memory serve directly. */
typedef struct akv_host_tier {
  const void* blocks;          /* 16-byte aligned */
  int32_t length;              /* tokens; must equal quant.lengths[b] on the device */
} akv_host_tier;

/* Staging for akv_attend_decode_staged.  The ring (device memory) is cut
 * into `slots` equal slots; each holds the blocks of one chunk of whole
 * compressed splits.  copy_stream and the 2*slots + 1 events are the
 * caller's (created with hipStreamCreate / hipEventCreate, default priority);
 * the library only enqueues on them. */
typedef struct akv_staging_desc {
  uint32_t struct_size;        /* sizeof(akv_staging_desc) */
  const akv_host_tier* seqs;   /* host array [B] */
  void* ring;                  /* device, 256-byte aligned */
  size_t ring_bytes;
  int32_t slots;               /* >= 2 */
  void* copy_stream;           /* hipStream_t of the host-to-device copies */
  void* const* events;         /* host array of 2*slots + 1 hipEvent_t */
} akv_staging_desc;

/* Split-KV decode attention, one query token per sequence (ActiveKV,
 * "Context beyond VRAM", "What I built": each tier of the history gives its
 * own partial result and the partials are joined by exact attention
 * arithmetic; the compressed tier is read through a query rotated once,
 * because the Hadamard rotation keeps dot products -- QuantForge walkthrough,
 * section 1, "Triton Fused Kernels"; each partial carries the log-sum-exp
 * statistic of "Bringing a serving stack up on new silicon", "What I built").
 * Enqueues two kernels: a split kernel in which every (split, kv head,
 * sequence) workgroup attends its split (the compressed tier with the
 * pre-rotated query and the value sum kept in rotated space) and writes a
 * partial, then a merge kernel that, per (sequence, query head), merges the
 * compressed-tier partials, inverse-rotates once and merges with the
 * exact-tier partials.  The merge uses a fixed reduction tree, so repeated
 * calls give identical bytes.  ws (scratch for the partials; no state is
 * kept between calls) must be 256-byte aligned and at least
 * akv_decode_workspace_bytes(desc) bytes; calls that overlap in time on one
 * workspace race. */
akv_status akv_attend_decode(const akv_attn_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* akv_attend_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * hipMalloc): no workspace argument; the partials live in the library's own
 * device array of AKV_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until
 * the process ends.  Same validation, kernels and results as
 * akv_attend_decode (bit for bit); a shape whose workspace
 * (akv_decode_workspace_bytes) exceeds the array returns AKV_ERR_WORKSPACE.
 * The call allocates nothing.  Its first call on a GPU looks up that GPU's
 * array (a HIP symbol query, AKV_ERR_HIP if it fails).  Every call on one GPU
 * shares that GPU's array, and nothing in it must start at zero (each call
 * writes every value it reads): calls that overlap in time on one GPU race,
 * so serialize them (one stream, or events). */
#define AKV_NOALLOC_SCRATCH_BYTES (64u << 20)
akv_status akv_attend_decode_noalloc(const akv_attn_desc* desc, void* stream);

/* akv_attend_decode with the compressed tier streamed from pinned host memory
 * (ActiveKV, "Context beyond VRAM", "What I built": host memory owns the
 * history, device memory holds a bounded staging area, and no staged bytes
 * are overwritten while a kernel may still read them).  The exact tier and the query are on the device as in
 * akv_attend_decode; desc->quant supplies lengths (device, for the merge) and
 * max_blocks (the split plan), and its pools and table may be NULL.  Per
 * sequence, runs of whole compressed splits (their records, one
 * hipMemcpyAsync each) are copied on copy_stream into the next ring slot
 * while earlier slots are attended on
 * `stream`; events order each copy after the kernel that last read its slot
 * and each kernel after its copy.  Same splits, same arithmetic and same
 * merge as akv_attend_decode, so the outputs are bit-identical to it.  A
 * ring too small for one split of every tier block size returns
 * AKV_ERR_WORKSPACE. */
akv_status akv_attend_decode_staged(const akv_attn_desc* desc, const akv_staging_desc* staging, void* ws,
                                    size_t ws_bytes, void* stream);

/* Prefill-chunk attention: Tq causal queries per sequence over the two-tier
 * history (the prefill side of ActiveKV's two-tier cache; causal rule in the
 * akv_attn_desc comment).  Enqueues two kernels (three with a given
 * rotation: the queries are rotated by R first): a split kernel on 16x16x32
 * matrix-core tiles in which every (128 (query, head) rows of a kv head,
 * split, sequence) workgroup expands each block of its split into LDS once
 * (compressed K as fp16 hi + lo parts against a hi + lo rotated query; exact
 * K/V as bf16) and writes one partial per row, then a merge kernel that per
 * (sequence, query, head) merges the partials in ascending split order,
 * inverse-rotates the compressed-tier result once (R^T with a given
 * rotation) and merges the tiers.  Every code width of "Code width" is
 * served.  Repeated calls give identical bytes.  A sequence whose exact length is
 * below Tq (the chunk must be in the exact tier) or whose lengths are out of
 * range gets NaN outputs.  ws as for decode, with
 * akv_chunk_workspace_bytes(desc) bytes. */
akv_status akv_attend_chunk(const akv_attn_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* Exact log-sum-exp merge of P normalized partials of R rows of width d (the
 * per-row log-sum-exp that "Bringing a serving stack up on new silicon",
 * "What I built", adds to paged attention is what lets partial results over
 * disjoint pieces of a history be joined exactly, as ActiveKV joins its two
 * tiers -- "Context beyond VRAM", "What I built"):
 * o_parts [P][R][d], lse_parts [P][R] (natural log), outputs o_out [R][d],
 * lse_out [R].  Per row: M = max_p lse_p; if M = -inf the row is empty and
 * gets o = 0, lse = -inf; else w_p = exp(lse_p - M), W = sum_p w_p,
 * lse = M + ln W and o = sum_p (w_p / W) o_p, summed in ascending p.  NaN
 * inputs propagate; +inf is invalid input.  1 <= P <= 4096, 1 <= d <= 1024,
 * all pointers 4-byte aligned. */
akv_status akv_lse_merge(const float* o_parts, const float* lse_parts, int32_t P, int32_t R,
                         int32_t d, float* o_out, float* lse_out, void* stream);

/* Compress evicted exact-tier tokens into the compressed tier (see
 * akv_compress_desc).  Enqueues one encode kernel. */
akv_status akv_compress_evicted(const akv_compress_desc* desc, void* stream);

/* One decode step's history bookkeeping, fused on the GPU (ActiveKV,
 * "Context beyond VRAM", "What I built": each step appends the new key/value
 * to the recent exact window, and older history lives in the compact tier).
 * For every sequence b, with n = exact_lengths[b] and m = quant_lengths[b]
 * read on the device:
 *   1. the new token's K and V (bf16 [B][Hkv][d]) are written at exact-tier
 *      position n (block exact_table[b][n / 64], layouts above);
 *   2. if n + 1 >= window + 64 and m + 64 <= 64 * quant_max_blocks (any m,
 *      even or odd), the 64 oldest exact tokens (the first block of the row) are rotated
 *      and encoded into compressed positions [m, m + 64) exactly as
 *      akv_compress_evicted encodes them, the ceil((n + 1) / 64) entries in
 *      use of the exact table row rotate left by one (the freed block comes
 *      right after the blocks still in use, where the appends continue),
 *      exact_lengths[b] = n + 1 - 64 and quant_lengths[b] = m + 64;
 *   3. otherwise exact_lengths[b] = n + 1.
 * Lengths and the exact table are device memory, updated in place; the
 * compressed table is only read.  A sequence whose exact table has no room
 * for the new token (n / 64 >= exact_max_blocks), or whose length is out of
 * range, gets exact_lengths[b] = -1, so its attention outputs are NaN until
 * the caller resets it.  window: a positive multiple of 64 with
 * window / 64 + 1 <= exact_max_blocks.  Enqueues two kernels (append +
 * encode, then lengths and table).  Calls on one sequence must not overlap. */
typedef struct akv_append_desc {
  uint32_t struct_size;        /* sizeof(akv_append_desc) */
  int32_t B, Hkv, d, window;
  const uint16_t* new_k;       /* bf16 [B][Hkv][d], 16-byte aligned */
  const uint16_t* new_v;
  uint16_t* exact_k;           /* exact-tier pools (layouts above) */
  uint16_t* exact_v;
  int32_t* exact_table;        /* [B][exact_max_blocks], rotated in place */
  int32_t* exact_lengths;      /* [B], updated in place */
  int32_t exact_max_blocks, exact_num_blocks;
  uint8_t* k_codes;            /* compressed-tier pools (layouts above) */
  uint8_t* v_codes;
  uint16_t* k_scales;
  uint16_t* v_scales;
  const int32_t* quant_table;  /* [B][quant_max_blocks] */
  int32_t* quant_lengths;      /* [B], updated in place */
  int32_t quant_max_blocks, quant_num_blocks;
  const float* rotation;       /* NULL, or the rotation R (see "Rotation") */
  int32_t code_bits;           /* 0 or 4, 3, 2 (see "Code width") */
} akv_append_desc;

akv_status akv_append_evict(const akv_append_desc* desc, void* stream);

/* Context checkpoint (ActiveKV, "Context beyond VRAM", "What I built": a
 * context can be parked and brought back later without being rebuilt from its
 * tokens).  The image of a
 * batch is a fixed-size byte string, every field little-endian:
 *   [0, 256)   header: "AKVCTX01" (8 bytes), then int32 B, Hkv, d,
 *              exact_max_blocks, quant_max_blocks, code width w (2, 3
 *              or 4), zeros up to 256;
 *   [256, 256 + 8B) int32 exact_lengths[b], quant_lengths[b] for b = 0..B-1,
 *              zeros up to the next multiple of 256 (offset E);
 *   at E:      for b, then slot j < exact_max_blocks: the exact block of
 *              tokens [64j, 64j + 64) as Hkv K slabs then Hkv V slabs
 *              (256*Hkv*d bytes, pool layouts above);
 *   then:      for b, then slot j < quant_max_blocks: K codes, V codes
 *              (8*w*d*Hkv bytes each), K scales, V scales (4*d*Hkv bytes
 *              each).
 * Slots at or past ceil(length / 64) are zeros, as are the bytes of a slot
 * whose table entry is outside [0, num_blocks).  The image depends only on
 * the tokens (not on which pool blocks hold them), so a context restored into
 * another block placement attends bit-identically. */
typedef struct akv_context_desc {
  uint32_t struct_size;        /* sizeof(akv_context_desc) */
  int32_t B, Hkv, d;
  uint16_t* exact_k;           /* exact-tier pools (layouts above) */
  uint16_t* exact_v;
  const int32_t* exact_table;  /* [B][exact_max_blocks] */
  int32_t* exact_lengths;      /* [B] */
  int32_t exact_max_blocks, exact_num_blocks;
  uint8_t* k_codes;            /* compressed-tier pools (layouts above) */
  uint8_t* v_codes;
  uint16_t* k_scales;
  uint16_t* v_scales;
  const int32_t* quant_table;  /* [B][quant_max_blocks] */
  int32_t* quant_lengths;      /* [B] */
  int32_t quant_max_blocks, quant_num_blocks;
  int32_t code_bits;           /* 0 or 4, 3, 2 (see "Code width") */
} akv_context_desc;

/* Bytes of the image for desc's shape; 0 if desc is invalid. */
size_t akv_checkpoint_bytes(const akv_context_desc* desc);

/* Write the image of the batch into `image` (any memory the device can write:
 * HBM, or mapped pinned host memory; 256-byte aligned, at least
 * akv_checkpoint_bytes(desc) bytes).  Reads the pools, tables and lengths;
 * writes nothing else.  One gather kernel. */
akv_status akv_checkpoint_save(const akv_context_desc* desc, void* image, void* stream);

/* Restore an image into the pool blocks that desc's tables name (which may
 * differ from the saved placement): the slots below each saved length are
 * copied to their blocks, then the lengths are set.  An image whose header
 * does not match desc's shape, or a table entry outside [0, num_blocks),
 * sets that batch's (or sequence's) exact length to -1, so its attention is
 * NaN.  One scatter kernel; desc's pools, tables and lengths must not be in
 * use by other work while it runs. */
akv_status akv_checkpoint_restore(const akv_context_desc* desc, const void* image, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* AKV_H */
