/*
 * tq_decode.h -- C ABI of the MI355X (gfx950) paged grouped-query decode
 * attention library (libtqdecode.so).
 *
 * One decode step of attention for every sequence of a batch: each sequence
 * has ONE new query token with Hq = Hkv * QG query heads (grouped-query
 * attention: query heads h*QG .. h*QG+QG-1 share kv head h) and attends to
 * its L cached tokens, which live in a paged KV cache addressed through a
 * block table.  The context is split into partitions of E = 256 * G tokens
 * (flash-decoding split-K); tq_decode computes one normalised partial result
 * per live partition and tq_decode_reduce merges the partials by log-sum-exp.
 * Page "vllm.v1.attention.ops.flydsl_kernels.tq_decode": the argument list,
 * supported sizes and partition semantics are those of the docstring of
 * build_tq_decode_module; the partial triple (out, exp_sums, max_logits) is
 * that of STEP G of tq_decode_kernel.
 *
 * Cache format.  The page's 4-bit "TQ" contents are left open there; this
 * library stores K and V as OCP fp8 e4m3fn codes with one fp32 scale per
 * (token, kv head) for K and one for V (or, second format, the 4-bit record
 * below).  The scales are SoA metadata per cache block in the kv_head ->
 * field -> slot order of the page's per-block metadata region.  The 128-byte
 * code rows of a block are in one of two orders, chosen by ext->kv_layout:
 *   TQ_KV_LAYOUT_SLOT_MAJOR: the page's data region (STEP F of
 *     tq_decode_kernel: slot stride num_kv_heads rows, kv head stride one row)
 *     k_cache, v_cache : uint8 [num_blocks][BS][Hkv][128]   (e4m3fn codes)
 *   TQ_KV_LAYOUT_HEAD_MAJOR (0, the default): the BS rows of one (block, kv
 *     head) are one contiguous 2 or 4 KiB range, which streams faster
 *     k_cache, v_cache : uint8 [num_blocks][Hkv][BS][128]
 *   kv_scales          : fp32  [num_blocks][Hkv][2][BS]     (field 0 = K, 1 = V)
 * The dequantized value is code * scale (scales of either sign).
 *
 * Memory and threading.
 *   - Every pointer argument is a DEVICE pointer (HIP device memory) owned
 *     by the caller, except `ext` and `partials`, which point to HOST structs
 *     read during the call only.  The library allocates nothing, keeps no
 *     state other than a thread-local last HIP error (and, for
 *     tq_decode_fused_static only, its static scratch), never synchronizes, and
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *     stream).  All calls are asynchronous and reentrant.
 *   - q, k_cache, v_cache, kv_scales, the partial buffers and out must be
 *     16-byte aligned.
 *   - Argument errors are detected on the host before anything is enqueued;
 *     the call then returns the status and the device is not touched.  A
 *     failed launch returns TQ_ERR_HIP (see tq_last_hip_error()).  Faults of
 *     an enqueued kernel surface at the caller's next synchronization.
 *   - Device-side values are clamped, never trusted for addressing: a
 *     seq_lens entry is clamped to [0, min(max_seq_len_bound, P*E,
 *     max_blocks_per_seq*BS)] where max_seq_len_bound = ext->max_seq_len, and
 *     a block-table entry to [0, num_blocks-1].  A caller that breaks the
 *     contract (a length above ext->max_seq_len, a block id outside the
 *     pool) gets wrong numbers, never an out-of-bounds access.
 *   - Debugging such a caller: with TQ_VALIDATE=1 in the environment (read on
 *     every call), each decode entry point first enqueues a check kernel that
 *     prints, by device printf, every sequence whose length is outside [0,
 *     ext->max_seq_len] and the first block-table entry of each sequence that
 *     is outside [0, num_blocks) for a token below its length.  The decode
 *     then runs as always (clamped).  Off by default; for debugging only.
 */
#ifndef TQ_DECODE_H
#define TQ_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 2
#define TQ_HEAD_DIM 128
#define TQ_TOKENS_PER_TILE_GROUP 256 /* 16 tiles of 16 tokens */
/* Device memory per GPU of tq_decode_fused_static's scratch, and its counter region. */
#define TQ_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
#define TQ_STATIC_COUNTER_BYTES ((size_t)1 << 20)

typedef enum {
  TQ_OK = 0,
  TQ_ERR_NULL = 1,        /* a required pointer is NULL */
  TQ_ERR_MISALIGNED = 2,  /* a data pointer is not 16-byte aligned */
  TQ_ERR_UNSUPPORTED = 3, /* QG not in {6, 8, 16}, BS not in {16, 32}, head_dim != 128,
                             or an unknown kv_layout */
  TQ_ERR_SHAPE = 4,       /* num_seqs, Hkv, num_blocks, max_blocks_per_seq, P or G < 1,
                             or a size that overflows the index types */
  TQ_ERR_COVERAGE = 5,    /* max_seq_len < 0, > P*G*256 or > max_blocks_per_seq*BS */
  TQ_ERR_SCALE = 6,       /* softmax_scale not finite or <= 0 */
  TQ_ERR_HIP = 7,         /* a HIP launch failed; see tq_last_hip_error() */
  TQ_ERR_SCRATCH = 8      /* tq_decode_fused_static: the batch needs more than the static
                             scratch holds */
} tq_status;

/* Order of the 128-byte K / V rows inside a cache block (tq_extent.kv_layout;
 * tq_kv_write's kv_layout); anything else is TQ_ERR_UNSUPPORTED. */
#define TQ_KV_LAYOUT_HEAD_MAJOR 0 /* [Hkv][BS] rows */
#define TQ_KV_LAYOUT_SLOT_MAJOR 1 /* [BS][Hkv] rows: the page's data region */

/* Sizes that a decode step needs besides the named arguments (host struct). */
typedef struct {
  int32_t num_seqs;           /* S: sequences in the batch (>= 1) */
  int32_t num_blocks;         /* NB: physical blocks in k_cache / v_cache / kv_scales (>= 1) */
  int32_t max_blocks_per_seq; /* row length (stride) of block_tables (>= 1) */
  int32_t num_partitions;     /* P: partitions per (sequence, kv head) (>= 1) */
  int32_t max_seq_len;        /* host-known upper bound of seq_lens[] (0 <= . <= P*E) */
  int32_t head_dim;           /* must be 128 */
  int32_t kv_layout;          /* TQ_KV_LAYOUT_HEAD_MAJOR (0) or TQ_KV_LAYOUT_SLOT_MAJOR */
} tq_extent;

/* The split-K partial triple (host struct of device pointers), fp32:
 *   out        [S][Hkv][P][QG][128]  partial output o_p, normalised by its own l_p
 *   max_logits [S][Hkv][P][QG]       m_p = max over the partition's tokens of the
 *                                    scaled logit x = softmax_scale * q.k (natural-log units)
 *   exp_sums   [S][Hkv][P][QG]       l_p = sum over those tokens of exp(x - m_p)
 * Entries are written only for live partitions (p*E < L); others are left untouched. */
typedef struct {
  float* out;
  float* max_logits;
  float* exp_sums;
} tq_partials;

/*
 * tq_decode -- the partition kernel: for every (sequence s, kv head h,
 * partition p) with p*E < L_s, where E = 256 * tile_groups_per_partition,
 * attend the QG query rows q[s][h*QG + g] to the cached tokens
 * [p*E, min((p+1)*E, L_s)) and write the partial triple.
 *   q              bf16 [S][Hkv*QG][128]
 *   k_cache        e4m3fn [NB][Hkv][BS][128], or [NB][BS][Hkv][128] (ext->kv_layout)
 *   v_cache        e4m3fn, the same layout as k_cache
 *   kv_scales      fp32 [NB][Hkv][2][BS]
 *   block_tables   int32 [S][max_blocks_per_seq]: token t of sequence s is slot
 *                  t % BS of block block_tables[s][t / BS]; entries at or past
 *                  ceil(L_s / BS) are never read
 *   seq_lens       int32 [S]: L_s
 *   partials       where the partial triple goes (see tq_partials)
 *   num_kv_heads   Hkv >= 1
 *   query_group_size  QG in {6, 8, 16}
 *   kv_block_size  BS in {16, 32}
 *   tile_groups_per_partition  G >= 1 (E = 256 * G tokens per partition)
 *   softmax_scale  finite and > 0 (1/sqrt(128) is the usual value)
 *   ext, stream    see above
 * Cache slots at or past L_s may hold any bytes (NaN codes and scales
 * included); they never change the result.
 */
tq_status tq_decode(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                    const float* kv_scales, const int32_t* block_tables, const int32_t* seq_lens,
                    const tq_partials* partials, int32_t num_kv_heads, int32_t query_group_size,
                    int32_t kv_block_size, int32_t tile_groups_per_partition, float softmax_scale,
                    const tq_extent* ext, void* stream);

/*
 * tq_decode_reduce -- the merge kernel: for every (s, h, g), over the live
 * partitions p of sequence s, M = max m_p, w_p = l_p * exp(m_p - M) and
 *   out[s][h*QG + g][:] = bf16_rne( sum_p (w_p / sum_p' w_p') * o_p )
 * With a single live partition this is exactly bf16_rne(o_0); L_s = 0 gives
 * zeros.  The merge itself is not on the page; it is the log-sum-exp
 * combination that the partial triple of STEP G of tq_decode_kernel implies.
 *   out  bf16 [S][Hkv*QG][128], fully overwritten.
 * The other arguments mean what they mean for tq_decode and must be the same
 * values that produced the partials.
 */
tq_status tq_decode_reduce(const tq_partials* partials, const int32_t* seq_lens, void* out,
                           int32_t num_kv_heads, int32_t query_group_size,
                           int32_t tile_groups_per_partition, const tq_extent* ext, void* stream);

/*
 * tq_decode_fused -- the whole decode step in one launch, bf16 out directly.
 * With a large enough workspace (tq_fused_workspace_bytes) and at most 1024
 * sequences, the live 32-token chunks of all (sequence s, kv head h) pairs
 * form one list in (s, h, chunk) order, dealt evenly to the waves of one
 * resident round of workgroups (8 waves each): every wave streams the same
 * number of chunks to within one, however ragged the lengths.  Each
 * wave keeps one online softmax per (s, h) it touches; the partial results (o,
 * m, l, as in STEP G of tq_decode_kernel) of an (s, h) split across waves are
 * merged by log-sum-exp with the formula of tq_decode_reduce, first in LDS
 * among the waves of a workgroup, then, for an (s, h) split across
 * workgroups, through `workspace`: the last workgroup to finish merges them in
 * workgroup order and writes out.  This is the in-launch merge across
 * partitions that the page's partial triple implies, with no second launch.
 * Without a workspace (or with more than 1024 sequences, or too few bytes)
 * each (s, h) gets its own workgroups instead, its tile groups (256 tokens,
 * the page's unit of work) dealt in contiguous runs to them, with the same
 * merges.
 *   out        bf16 [S][Hkv*QG][128], fully overwritten (L_s = 0 gives zeros)
 *   workspace  NULL, or device memory of workspace_bytes bytes, 16-byte
 *              aligned; ZERO-FILLED before its first use.  Its first
 *              round_up(4 * S * Hkv, 256) bytes hold arrival counters that every
 *              call leaves at zero again; the partials follow them, so a call
 *              with another S * Hkv would find its counters where an earlier
 *              call left partials: reuse a workspace only for calls with the
 *              same num_seqs and num_kv_heads, or zero-fill it again first.
 *              Calls that run concurrently must not share a workspace.
 * tile_groups_per_partition and ext->num_partitions bound the context as for
 * tq_decode (coverage check); the split itself is the library's choice: a
 * function of the sizes, ext->max_seq_len, workspace_bytes and the device-side
 * lengths, so repeated calls are bit-identical, and one launch serves any
 * lengths up to ext->max_seq_len (a captured graph may be replayed with new
 * lengths).  An (s, h) that one wave computes whole (L <= 32 with the list,
 * L <= 256 with per-(s, h) workgroups) is bit-identical to tq_decode +
 * tq_decode_reduce; otherwise the two paths differ only by rounding.  Other
 * arguments and errors are those of tq_decode.
 */
tq_status tq_decode_fused(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                          const float* kv_scales, const int32_t* block_tables,
                          const int32_t* seq_lens, void* out, int32_t num_kv_heads,
                          int32_t query_group_size, int32_t kv_block_size,
                          int32_t tile_groups_per_partition, float softmax_scale,
                          const tq_extent* ext, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * tq_decode_fused_static -- tq_decode_fused for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc): the same decode, with the library's own static
 * scratch in place of the caller's workspace.  The split, and so every output
 * bit, is the one tq_decode_fused takes with a zero-filled workspace of
 * tq_fused_workspace_bytes() bytes.
 *   Scratch: TQ_STATIC_SCRATCH_BYTES (8 MiB) of device memory per GPU that the
 *   library runs on, held until the process ends: arrival counters in the
 *   first TQ_STATIC_COUNTER_BYTES (1 MiB, 4 B per (s, h)), workgroup partials
 *   after them.  Its device address is taken once per GPU, on the first call
 *   on it (the calling thread's current device must be the one `stream`
 *   belongs to); that call also enqueues the scratch's zero fill on `stream`.
 *   Every call leaves the counters at zero; the partials keep the last call's
 *   contents.  All calls on one GPU share its scratch: calls that overlap in
 *   time on one GPU (other streams, other threads) race and give wrong results.
 *   This entry point allocates nothing and frees nothing.
 *   Returns TQ_ERR_SCRATCH, before anything is enqueued, when the batch needs
 *   more than the scratch holds: more than 262144 (sequence, kv head) pairs,
 *   or more than 7 MiB of partials (the even split needs at most 4.1 MiB).
 * Other arguments and errors are those of tq_decode_fused.
 */
tq_status tq_decode_fused_static(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                 const float* kv_scales, const int32_t* block_tables,
                                 const int32_t* seq_lens, void* out, int32_t num_kv_heads,
                                 int32_t query_group_size, int32_t kv_block_size,
                                 int32_t tile_groups_per_partition, float softmax_scale,
                                 const tq_extent* ext, void* stream);

/* Workspace bytes for the fastest split of tq_decode_fused at these sizes on a
 * device of 256 compute units, the largest split the library plans (a device
 * with fewer CUs uses fewer of them; 0: it needs none).  Depends on num_seqs, max_seq_len, num_kv_heads and
 * query_group_size: with the even split, 256 B-rounded arrival counters (4 B per
 * (s, h)) and two partial slots per workgroup (QG*520 B each). */
size_t tq_fused_workspace_bytes(const tq_extent* ext, int32_t num_kv_heads,
                                int32_t query_group_size);

/*
 * The 4-bit record format -- the "TQ" cache of page "vllm.v1.attention.ops.
 * flydsl_kernels.tq_decode" (STEP F: K dequantized as centroids[index] * K
 * norm, V as index * V scale + V zero point; the query rotated by the caller).
 * The page leaves the record's constants open; this library reads them as:
 *   kv_cache   uint8 [NB][tq4_block_bytes(Hkv, BS)], one cache block =
 *              data rows of 128 bytes, [BS][Hkv] (TQ_KV_LAYOUT_SLOT_MAJOR:
 *              the page's data region, STEP F) or [Hkv][BS]
 *              (TQ_KV_LAYOUT_HEAD_MAJOR, the default): per (kv head, slot) the
 *              K indices in bytes 0..63 and the V indices in bytes 64..127,
 *              dim d in byte d/2, low nibble for even d, high nibble for odd d;
 *              then metadata [Hkv][3][BS] IEEE fp16: field 0 = K norm, 1 = V
 *              scale, 2 = V zero point.  16-byte aligned.
 *   centroids  fp32 [16], the K codebook.  4-byte aligned.
 *   q_rot      bf16 [S][Hkv*QG][128], the query in the rotated basis of K.
 * k_t[d] = centroids[kidx] * knorm_t, v_t[d] = vidx * vscale_t + vzero_t, and
 * the attention is the one of tq_decode.  Records past a sequence's length may
 * hold any bytes (NaN metadata included).
 *
 * tq4_decode writes the same partial triple as tq_decode (merge it with
 * tq_decode_reduce); tq4_decode_fused is tq_decode_fused for this format (the
 * workspace size is tq_fused_workspace_bytes).  Arguments, checks and errors
 * are those of tq_decode / tq_decode_fused, with kv_cache and centroids in
 * place of k_cache, v_cache and kv_scales.
 */
tq_status tq4_decode(const void* q_rot, const uint8_t* kv_cache, const float* centroids,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const tq_partials* out, int32_t num_kv_heads, int32_t query_group_size,
                     int32_t kv_block_size, int32_t tile_groups_per_partition, float softmax_scale,
                     const tq_extent* ext, void* stream);
tq_status tq4_decode_fused(const void* q_rot, const uint8_t* kv_cache, const float* centroids,
                           const int32_t* block_tables, const int32_t* seq_lens, void* out,
                           int32_t num_kv_heads, int32_t query_group_size, int32_t kv_block_size,
                           int32_t tile_groups_per_partition, float softmax_scale,
                           const tq_extent* ext, void* workspace, size_t workspace_bytes,
                           void* stream);
/* Bytes of one 4-bit cache block: Hkv*BS*128 + Hkv*3*BS*2 (0 if BS is unsupported). */
size_t tq4_block_bytes(int32_t num_kv_heads, int32_t kv_block_size);

/*
 * tq_kv_write -- the KV-cache writer, the step that fills the cache the
 * decode reads: for each new token t with 0 <= slot_mapping[t] < NB*BS
 * (slot = block * BS + offset) and each kv head h, the K row and the V row are
 * quantized on their own,
 *   s = fp32(absmax / 448),  code_d = e4m3fn(x_d / s)
 * (fp32 division, round to nearest even, saturating at +-448; an all-zero row
 * gives s = 0 and codes 0), and stored in the row of (block, h, offset) of
 * k_cache / v_cache, in the row order kv_layout names (as for tq_decode:
 * [NB][Hkv][BS][128] or [NB][BS][Hkv][128]), with s at
 * kv_scales[block][h][0 or 1][offset].  Other slots are untouched;
 * a negative slot (padding) or one at or past NB*BS is skipped.  The
 * per-block scale region follows the fp8 record writer of page
 * "vllm.models.deepseek_v41.amd.mono.attention.front" (stage_qkv), with this
 * library's scale rule instead of its power-of-two scale codes.
 *   k_new, v_new   bf16 [T][Hkv][128], finite values
 *   slot_mapping   int32 [T]
 *   k_cache, v_cache, kv_scales   as for tq_decode (written in place)
 *   kv_layout      TQ_KV_LAYOUT_HEAD_MAJOR or TQ_KV_LAYOUT_SLOT_MAJOR
 * Tokens that map to the same slot race: the caller must not do that.
 * Errors as for tq_decode; num_tokens = 0 is a no-op.
 */
tq_status tq_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                      uint8_t* k_cache, uint8_t* v_cache, float* kv_scales, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t kv_block_size, int32_t num_blocks,
                      int32_t head_dim, int32_t kv_layout, void* stream);

/* Bytes of the three partial arrays for these sizes (each rounded up to 256 B),
 * laid out out | max_logits | exp_sums; 0 if the sizes are invalid. */
size_t tq_partials_bytes(const tq_extent* ext, int32_t num_kv_heads, int32_t query_group_size);

/* Static, human-readable text for a status code. */
const char* tq_status_str(tq_status status);

/* hipError_t of the last TQ_ERR_HIP returned on the calling thread (0 if none). */
int32_t tq_last_hip_error(void);

/* TQ_ABI_VERSION of the loaded library. */
int32_t tq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_DECODE_H */
