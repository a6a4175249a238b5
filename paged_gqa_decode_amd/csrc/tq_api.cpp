// C ABI of libtqdecode.so (declared in include/tq_decode.h): host-side
// argument checks, sizes and kernel dispatch.  Nothing here touches the
// device before every check has passed.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "tq_decode.h"
#include "tq_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

bool supported_qg(int32_t qg) { return qg == 6 || qg == 8 || qg == 16; }
bool supported_bs(int32_t bs) { return bs == 16 || bs == 32; }

// Byte distances between the 128-byte rows of consecutive kv heads and slots
// inside a cache block, for either row order.
void set_row_strides(int32_t layout, int32_t num_kv_heads, int32_t kv_block_size,
                     int32_t* head_stride, int32_t* slot_stride) {
  if (layout == TQ_KV_LAYOUT_SLOT_MAJOR) {
    *head_stride = TQ_HEAD_DIM;
    *slot_stride = num_kv_heads * TQ_HEAD_DIM;
  } else {
    *head_stride = kv_block_size * TQ_HEAD_DIM;
    *slot_stride = TQ_HEAD_DIM;
  }
}

// Checks shared by both entry points.  On success fills partition_tokens and
// len_cap (the device-side clamp of sequence lengths).
tq_status check_common(const tq_extent* ext, int32_t num_kv_heads, int32_t query_group_size,
                       int32_t tile_groups_per_partition, int32_t* partition_tokens) {
  if (!ext) return TQ_ERR_NULL;
  if (ext->head_dim != TQ_HEAD_DIM || !supported_qg(query_group_size)) return TQ_ERR_UNSUPPORTED;
  if (ext->num_seqs < 1 || num_kv_heads < 1 || ext->num_blocks < 1 || ext->max_blocks_per_seq < 1 ||
      ext->num_partitions < 1 || tile_groups_per_partition < 1)
    return TQ_ERR_SHAPE;
  const int64_t E = (int64_t)TQ_TOKENS_PER_TILE_GROUP * tile_groups_per_partition;
  const int64_t units = (int64_t)ext->num_seqs * num_kv_heads * ext->num_partitions;
  if (E > INT32_MAX / 2 || units > INT32_MAX || (int64_t)ext->num_seqs * num_kv_heads > INT32_MAX)
    return TQ_ERR_SHAPE;
  if ((int64_t)ext->num_partitions * E > INT32_MAX) return TQ_ERR_SHAPE;
  if (ext->max_seq_len < 0 || (int64_t)ext->max_seq_len > (int64_t)ext->num_partitions * E)
    return TQ_ERR_COVERAGE;
  *partition_tokens = (int32_t)E;
  return TQ_OK;
}

// Checks of the decode arguments shared by tq_decode and tq_decode_fused
// (all but the output pointers); fills the stream arguments and E.
tq_status check_decode(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                       const float* kv_scales, const int32_t* block_tables,
                       const int32_t* seq_lens, int32_t num_kv_heads, int32_t query_group_size,
                       int32_t kv_block_size, int32_t tile_groups_per_partition,
                       float softmax_scale, const tq_extent* ext, tq::StreamArgs* st,
                       int32_t* E) {
  if (!q || !k_cache || !v_cache || !kv_scales || !block_tables || !seq_lens || !ext)
    return TQ_ERR_NULL;
  if (!supported_bs(kv_block_size)) return TQ_ERR_UNSUPPORTED;
  tq_status s = check_common(ext, num_kv_heads, query_group_size, tile_groups_per_partition, E);
  if (s != TQ_OK) return s;
  if ((int64_t)ext->max_seq_len > (int64_t)ext->max_blocks_per_seq * kv_block_size)
    return TQ_ERR_COVERAGE;
  if ((int64_t)num_kv_heads * kv_block_size * (TQ_HEAD_DIM + 3 * 2) > INT32_MAX) return TQ_ERR_SHAPE;
  if (ext->kv_layout != TQ_KV_LAYOUT_HEAD_MAJOR && ext->kv_layout != TQ_KV_LAYOUT_SLOT_MAJOR)
    return TQ_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return TQ_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(kv_scales) ||
      !aligned4(block_tables) || !aligned4(seq_lens))
    return TQ_ERR_MISALIGNED;
  st->q = static_cast<const uint16_t*>(q);
  st->k = k_cache;
  st->v = v_cache;
  st->scales = kv_scales;
  st->tq4 = nullptr;
  st->centroids = nullptr;
  st->tq4_block_bytes = 0;
  set_row_strides(ext->kv_layout, num_kv_heads, kv_block_size, &st->row_head_stride,
                  &st->row_slot_stride);
  st->bt = block_tables;
  st->num_kv_heads = num_kv_heads;
  st->max_blocks = ext->max_blocks_per_seq;
  st->num_blocks = ext->num_blocks;
  st->qk_scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
  return TQ_OK;
}

// The same checks for the 4-bit record format (cache and centroids instead of
// k_cache, v_cache and kv_scales).
tq_status check_decode_tq4(const void* q_rot, const uint8_t* kv_cache, const float* centroids,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int32_t num_kv_heads, int32_t query_group_size, int32_t kv_block_size,
                           int32_t tile_groups_per_partition, float softmax_scale,
                           const tq_extent* ext, tq::StreamArgs* st, int32_t* E) {
  if (!kv_cache || !centroids) return TQ_ERR_NULL;
  // kv_cache stands in for the fp8 pointers: alignment and null checks alike.
  tq_status s = check_decode(q_rot, kv_cache, kv_cache, reinterpret_cast<const float*>(kv_cache),
                             block_tables, seq_lens, num_kv_heads, query_group_size, kv_block_size,
                             tile_groups_per_partition, softmax_scale, ext, st, E);
  if (s != TQ_OK) return s;
  if (!aligned4(centroids)) return TQ_ERR_MISALIGNED;
  const int64_t block_bytes = (int64_t)num_kv_heads * kv_block_size * (TQ_HEAD_DIM + 3 * 2);
  if (block_bytes > INT32_MAX) return TQ_ERR_SHAPE;
  st->k = st->v = nullptr;
  st->scales = nullptr;
  st->tq4 = kv_cache;
  st->centroids = centroids;
  st->tq4_block_bytes = (int32_t)block_bytes;
  return TQ_OK;
}

tq_status hip_status(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int32_t)e;
    return TQ_ERR_HIP;
  }
  return TQ_OK;
}

// The partition kernel of either format, after the checks.
// TQ_VALIDATE=1 in the environment (read on every call): before a decode,
// enqueue the check kernel that prints lengths outside [0, max_seq_len] and
// block-table entries outside [0, num_blocks) (device printf, debug only; the
// decode itself clamps both and proceeds).
hipError_t maybe_validate(const tq::StreamArgs& st, const int32_t* seq_lens, int32_t kv_block_size,
                          const tq_extent* ext, void* stream) {
  const char* v = getenv("TQ_VALIDATE");
  if (!v || v[0] != '1') return hipSuccess;
  tq::ValidateArgs a{};
  a.bt = st.bt;
  a.seq_lens = seq_lens;
  a.num_seqs = ext->num_seqs;
  a.max_blocks = ext->max_blocks_per_seq;
  a.num_blocks = ext->num_blocks;
  a.kv_block_size = kv_block_size;
  a.max_seq_len = ext->max_seq_len;
  return tq::launch_validate(a, static_cast<hipStream_t>(stream));
}

tq_status run_partition(const tq::StreamArgs& st, const int32_t* seq_lens,
                        const tq_partials* partials, int32_t query_group_size,
                        int32_t kv_block_size, int32_t E, const tq_extent* ext, bool tq4,
                        void* stream) {
  if (!aligned16(partials->out) || !aligned4(partials->max_logits) || !aligned4(partials->exp_sums))
    return TQ_ERR_MISALIGNED;
  tq::PartitionArgs a{};
  a.st = st;
  a.seq_lens = seq_lens;
  a.o = partials->out;
  a.ml = partials->max_logits;
  a.es = partials->exp_sums;
  a.num_partitions = ext->num_partitions;
  a.partition_tokens = E;
  a.parts_per_wave = 1;  // chosen by the launcher
  a.len_cap = ext->max_seq_len;
  const hipError_t v = maybe_validate(st, seq_lens, kv_block_size, ext, stream);
  if (v != hipSuccess) return hip_status(v);
  return hip_status(tq::launch_partition(a, ext->num_seqs, query_group_size, kv_block_size, tq4,
                                         static_cast<hipStream_t>(stream)));
}

// The fused decode of either format, after the checks: the even split when
// it applies and the workspace holds it, else workgroups per (s, h).
// counters > 0: the workspace's counters take a fixed region of that many bytes
// (the static scratch) instead of the first counter_bytes(S * Hkv).
tq_status run_fused(const tq::StreamArgs& st, const int32_t* seq_lens, void* out,
                    int32_t num_kv_heads, int32_t query_group_size, int32_t kv_block_size,
                    const tq_extent* ext, void* workspace, size_t workspace_bytes, bool tq4,
                    void* stream, size_t counters = 0) {
  if (!aligned16(out) || (workspace && !aligned16(workspace))) return TQ_ERR_MISALIGNED;
  const hipError_t v = maybe_validate(st, seq_lens, kv_block_size, ext, stream);
  if (v != hipSuccess) return hip_status(v);
  const int64_t seq_heads = (int64_t)ext->num_seqs * num_kv_heads;
  const int cus = tq::device_cu_count();
  const int flat_groups = tq::plan_flat_groups(ext->num_seqs, num_kv_heads, ext->max_seq_len,
                                               tq::kFlatUnitTokens, cus);
  const size_t cb = counters ? counters : tq::counter_bytes(seq_heads);
  const bool counters_fit = workspace && cb >= tq::counter_bytes(seq_heads) && workspace_bytes >= cb;
  if (flat_groups > 0 && counters_fit &&
      workspace_bytes - cb >= tq::flat_partial_bytes(flat_groups, query_group_size)) {
    tq::FlatArgs f{};
    f.st = st;
    f.seq_lens = seq_lens;
    f.out = static_cast<uint16_t*>(out);
    f.len_cap = ext->max_seq_len;
    f.num_seqs = ext->num_seqs;
    f.n_groups = flat_groups;
    tq::bind_flat_workspace(&f, workspace, seq_heads, query_group_size, counters);
    return hip_status(tq::launch_flat(f, query_group_size, kv_block_size, tq4,
                                      static_cast<hipStream_t>(stream)));
  }
  const tq::FusedPlan plan = tq::plan_fused(seq_heads, ext->max_seq_len, query_group_size,
                                            workspace ? workspace_bytes : 0, counters, cus);
  tq::FusedArgs a{};
  a.st = st;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.len_cap = ext->max_seq_len;
  a.splits = plan.splits;
  a.counters = nullptr;
  a.ws_o = a.ws_m = a.ws_l = nullptr;
  if (plan.splits > 1) tq::bind_fused_workspace(&a, workspace, seq_heads, query_group_size, counters);
  return hip_status(tq::launch_fused(a, ext->num_seqs, plan.waves, query_group_size, kv_block_size,
                                     tq4, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

tq_status tq_decode(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                    const float* kv_scales, const int32_t* block_tables, const int32_t* seq_lens,
                    const tq_partials* partials, int32_t num_kv_heads, int32_t query_group_size,
                    int32_t kv_block_size, int32_t tile_groups_per_partition, float softmax_scale,
                    const tq_extent* ext, void* stream) {
  if (!partials || !partials->out || !partials->max_logits || !partials->exp_sums)
    return TQ_ERR_NULL;
  tq::StreamArgs st{};
  int32_t E = 0;
  tq_status rc = check_decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, num_kv_heads,
                              query_group_size, kv_block_size, tile_groups_per_partition,
                              softmax_scale, ext, &st, &E);
  if (rc != TQ_OK) return rc;
  return run_partition(st, seq_lens, partials, query_group_size, kv_block_size, E, ext, false,
                       stream);
}

tq_status tq_decode_fused(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                          const float* kv_scales, const int32_t* block_tables,
                          const int32_t* seq_lens, void* out, int32_t num_kv_heads,
                          int32_t query_group_size, int32_t kv_block_size,
                          int32_t tile_groups_per_partition, float softmax_scale,
                          const tq_extent* ext, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!out) return TQ_ERR_NULL;
  tq::StreamArgs st{};
  int32_t E = 0;
  tq_status rc = check_decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, num_kv_heads,
                              query_group_size, kv_block_size, tile_groups_per_partition,
                              softmax_scale, ext, &st, &E);
  if (rc != TQ_OK) return rc;
  return run_fused(st, seq_lens, out, num_kv_heads, query_group_size, kv_block_size, ext,
                   workspace, workspace_bytes, false, stream);
}

static_assert(tq::kStaticScratchBytes == TQ_STATIC_SCRATCH_BYTES &&
                  tq::kStaticCounterBytes == TQ_STATIC_COUNTER_BYTES,
              "the header states the static scratch sizes");

tq_status tq_decode_fused_static(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                                 const float* kv_scales, const int32_t* block_tables,
                                 const int32_t* seq_lens, void* out, int32_t num_kv_heads,
                                 int32_t query_group_size, int32_t kv_block_size,
                                 int32_t tile_groups_per_partition, float softmax_scale,
                                 const tq_extent* ext, void* stream) {
  if (!out) return TQ_ERR_NULL;
  tq::StreamArgs st{};
  int32_t E = 0;
  tq_status rc = check_decode(q, k_cache, v_cache, kv_scales, block_tables, seq_lens, num_kv_heads,
                              query_group_size, kv_block_size, tile_groups_per_partition,
                              softmax_scale, ext, &st, &E);
  if (rc != TQ_OK) return rc;
  // The split tq_decode_fused takes with a workspace of tq_fused_workspace_bytes():
  // its counters must fit the fixed counter region, its partials the rest.
  const int64_t seq_heads = (int64_t)ext->num_seqs * num_kv_heads;
  const size_t need = tq_fused_workspace_bytes(ext, num_kv_heads, query_group_size);
  const size_t cb = tq::counter_bytes(seq_heads);
  const size_t partials = need > cb ? need - cb : 0;
  if (cb > tq::kStaticCounterBytes || partials > tq::kStaticScratchBytes - tq::kStaticCounterBytes)
    return TQ_ERR_SCRATCH;
  void* scratch = nullptr;
  const hipError_t e = tq::static_scratch(&scratch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e);
  return run_fused(st, seq_lens, out, num_kv_heads, query_group_size, kv_block_size, ext, scratch,
                   tq::kStaticCounterBytes + partials, false, stream, tq::kStaticCounterBytes);
}

tq_status tq4_decode(const void* q_rot, const uint8_t* kv_cache, const float* centroids,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const tq_partials* partials, int32_t num_kv_heads, int32_t query_group_size,
                     int32_t kv_block_size, int32_t tile_groups_per_partition, float softmax_scale,
                     const tq_extent* ext, void* stream) {
  if (!partials || !partials->out || !partials->max_logits || !partials->exp_sums)
    return TQ_ERR_NULL;
  tq::StreamArgs st{};
  int32_t E = 0;
  tq_status rc = check_decode_tq4(q_rot, kv_cache, centroids, block_tables, seq_lens, num_kv_heads,
                                  query_group_size, kv_block_size, tile_groups_per_partition,
                                  softmax_scale, ext, &st, &E);
  if (rc != TQ_OK) return rc;
  return run_partition(st, seq_lens, partials, query_group_size, kv_block_size, E, ext, true,
                       stream);
}

tq_status tq4_decode_fused(const void* q_rot, const uint8_t* kv_cache, const float* centroids,
                           const int32_t* block_tables, const int32_t* seq_lens, void* out,
                           int32_t num_kv_heads, int32_t query_group_size, int32_t kv_block_size,
                           int32_t tile_groups_per_partition, float softmax_scale,
                           const tq_extent* ext, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!out) return TQ_ERR_NULL;
  tq::StreamArgs st{};
  int32_t E = 0;
  tq_status rc = check_decode_tq4(q_rot, kv_cache, centroids, block_tables, seq_lens, num_kv_heads,
                                  query_group_size, kv_block_size, tile_groups_per_partition,
                                  softmax_scale, ext, &st, &E);
  if (rc != TQ_OK) return rc;
  return run_fused(st, seq_lens, out, num_kv_heads, query_group_size, kv_block_size, ext,
                   workspace, workspace_bytes, true, stream);
}

size_t tq4_block_bytes(int32_t num_kv_heads, int32_t kv_block_size) {
  if (num_kv_heads < 1 || !supported_bs(kv_block_size)) return 0;
  return (size_t)num_kv_heads * kv_block_size * (TQ_HEAD_DIM + 3 * 2);
}

size_t tq_fused_workspace_bytes(const tq_extent* ext, int32_t num_kv_heads,
                                int32_t query_group_size) {
  if (!ext || ext->num_seqs < 1 || num_kv_heads < 1 || !supported_qg(query_group_size) ||
      ext->max_seq_len < 0)
    return 0;
  // Sized for a device of kFlatGroupsMax (256) CUs, the most the plans use: a
  // device with fewer CUs plans fewer workgroups and needs no more bytes.
  const int64_t seq_heads = (int64_t)ext->num_seqs * num_kv_heads;
  const int flat_groups = tq::plan_flat_groups(ext->num_seqs, num_kv_heads, ext->max_seq_len);
  if (flat_groups > 0) return tq::flat_workspace_bytes(seq_heads, flat_groups, query_group_size);
  const tq::FusedPlan plan = tq::plan_fused(seq_heads, ext->max_seq_len, query_group_size, SIZE_MAX);
  return tq::fused_workspace_bytes(seq_heads, plan.splits, query_group_size);
}

tq_status tq_decode_reduce(const tq_partials* partials, const int32_t* seq_lens, void* out,
                           int32_t num_kv_heads, int32_t query_group_size,
                           int32_t tile_groups_per_partition, const tq_extent* ext, void* stream) {
  if (!partials || !partials->out || !partials->max_logits || !partials->exp_sums || !seq_lens ||
      !out || !ext)
    return TQ_ERR_NULL;
  int32_t E = 0;
  tq_status st = check_common(ext, num_kv_heads, query_group_size, tile_groups_per_partition, &E);
  if (st != TQ_OK) return st;
  if (!aligned16(partials->out) || !aligned4(partials->max_logits) ||
      !aligned4(partials->exp_sums) || !aligned4(seq_lens) || !aligned16(out))
    return TQ_ERR_MISALIGNED;
  tq::ReduceArgs a{};
  a.o = partials->out;
  a.ml = partials->max_logits;
  a.es = partials->exp_sums;
  a.seq_lens = seq_lens;
  a.out = static_cast<uint16_t*>(out);
  a.num_kv_heads = num_kv_heads;
  a.query_group_size = query_group_size;
  a.num_partitions = ext->num_partitions;
  a.partition_tokens = E;
  a.len_cap = ext->max_seq_len;
  return hip_status(
      tq::launch_reduce(a, ext->num_seqs * num_kv_heads, static_cast<hipStream_t>(stream)));
}

tq_status tq_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                      uint8_t* k_cache, uint8_t* v_cache, float* kv_scales, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t kv_block_size, int32_t num_blocks,
                      int32_t head_dim, int32_t kv_layout, void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 1) return TQ_ERR_SHAPE;
  if (head_dim != TQ_HEAD_DIM || !supported_bs(kv_block_size) ||
      (kv_layout != TQ_KV_LAYOUT_HEAD_MAJOR && kv_layout != TQ_KV_LAYOUT_SLOT_MAJOR))
    return TQ_ERR_UNSUPPORTED;
  if ((int64_t)num_blocks * kv_block_size > INT32_MAX ||
      (int64_t)num_tokens * num_kv_heads > INT32_MAX / 2 ||
      (int64_t)num_kv_heads * kv_block_size * TQ_HEAD_DIM > INT32_MAX)
    return TQ_ERR_SHAPE;
  if (num_tokens == 0) return TQ_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !kv_scales) return TQ_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      !aligned16(kv_scales) || !aligned4(slot_mapping))
    return TQ_ERR_MISALIGNED;
  tq::KvWriteArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.slot_mapping = slot_mapping;
  a.k = k_cache;
  a.v = v_cache;
  a.scales = kv_scales;
  set_row_strides(kv_layout, num_kv_heads, kv_block_size, &a.row_head_stride, &a.row_slot_stride);
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.kv_block_size = kv_block_size;
  a.num_slots = num_blocks * kv_block_size;
  return hip_status(tq::launch_kv_write(a, static_cast<hipStream_t>(stream)));
}

size_t tq_partials_bytes(const tq_extent* ext, int32_t num_kv_heads, int32_t query_group_size) {
  if (!ext || ext->head_dim != TQ_HEAD_DIM || !supported_qg(query_group_size)) return 0;
  if (ext->num_seqs < 1 || num_kv_heads < 1 || ext->num_partitions < 1) return 0;
  const uint64_t rows = (uint64_t)ext->num_seqs * num_kv_heads * ext->num_partitions * query_group_size;
  auto up = [](uint64_t x) { return (x + 255u) & ~(uint64_t)255u; };
  return (size_t)(up(rows * TQ_HEAD_DIM * 4) + 2 * up(rows * 4));
}

const char* tq_status_str(tq_status status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "a required pointer is NULL";
    case TQ_ERR_MISALIGNED: return "a data pointer is not 16-byte aligned";
    case TQ_ERR_UNSUPPORTED: return "unsupported size or layout (query_group_size in {6,8,16}, kv_block_size in {16,32}, head_dim 128, kv_layout 0 or 1)";
    case TQ_ERR_SHAPE: return "invalid or overflowing shape (a count < 1 or too large)";
    case TQ_ERR_COVERAGE: return "max_seq_len is negative or exceeds num_partitions*256*G or max_blocks_per_seq*kv_block_size";
    case TQ_ERR_SCALE: return "softmax_scale must be finite and > 0";
    case TQ_ERR_HIP: return "HIP launch failed (see tq_last_hip_error)";
    case TQ_ERR_SCRATCH: return "the batch needs more than the library's static scratch holds (tq_decode_fused_static)";
  }
  return "unknown status";
}

int32_t tq_last_hip_error(void) { return g_last_hip_error; }

int32_t tq_abi_version(void) { return TQ_ABI_VERSION; }

}  // extern "C"
