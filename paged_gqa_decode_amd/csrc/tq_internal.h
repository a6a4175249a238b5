// Internal interface between the C ABI (tq_api.cpp) and the gfx950 kernels
// (tq_kernels.hip).  Not installed; the public interface is include/tq_decode.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace tq {

constexpr int kHeadDim = 128;
constexpr int kTokensPerTileGroup = 256;

// The flat fused kernel: waves per workgroup, and the sequences its length
// scan handles (64 lanes x kFlatSlices).
constexpr int kFlatWaves = 8;
constexpr int kFlatSlices = 16;
constexpr int kFlatMaxSeqs = 64 * kFlatSlices;
// Workgroups of the flat kernels at most (one per CU, up to the 256 CUs of an
// MI355X in its single-partition mode), and per lane of a wave that walks them
// all.  The grid itself follows the device's CU count (device_cu_count).
constexpr int kFlatGroupsMax = 256;
constexpr int kFlatGroupsPerLane = kFlatGroupsMax / 64;
// Tokens per entry of the flat fused kernel's work list: one 32-token chunk,
// so that the list splits evenly over the waves even when the tile groups are
// few per wave (ragged and long-context batches).
constexpr int kFlatUnitTokens = 32;

// What every decode kernel reads to stream one (sequence, kv head).  The fp8
// format uses k, v and scales; the 4-bit record format tq4 and centroids.
struct StreamArgs {
  const uint16_t* q;        // bf16 [S][Hkv*QG][128]
  const uint8_t* k;         // e4m3fn, NB blocks of Hkv*BS rows of 128 bytes
  const uint8_t* v;         // e4m3fn, the same
  const float* scales;      // fp32 [NB][Hkv][2][BS]
  const uint8_t* tq4;       // 4-bit records [NB][tq4_block_bytes]
  const float* centroids;   // fp32 [16]
  int32_t tq4_block_bytes;  // Hkv*BS*128 + Hkv*3*BS*2
  // Byte distance between the 128-byte rows of consecutive kv heads and of
  // consecutive slots inside a block (both formats): head-major blocks
  // [Hkv][BS][128] have (BS*128, 128), slot-major ones [BS][Hkv][128] (the
  // page's data region) (128, Hkv*128).
  int32_t row_head_stride;
  int32_t row_slot_stride;
  const int32_t* bt;        // int32 [S][max_blocks]
  int32_t num_kv_heads;
  int32_t max_blocks;       // block-table row stride
  int32_t num_blocks;       // NB, for clamping block ids
  float qk_scale_log2;      // softmax_scale * log2(e)
};

struct PartitionArgs {
  StreamArgs st;
  const int32_t* seq_lens;   // int32 [S]
  float* o;                  // fp32 [S][Hkv][P][QG][128]
  float* ml;                 // fp32 [S][Hkv][P][QG]
  float* es;                 // fp32 [S][Hkv][P][QG]
  int32_t num_partitions;
  int32_t partition_tokens;  // E = 256 * G
  int32_t parts_per_wave;    // consecutive partitions of one (s, h) walked by one wave
  int32_t len_cap;           // device lengths are clamped to [0, len_cap]
  int32_t num_seqs;          // S
  int32_t nt_partials;       // 1: partials stored with the non-temporal bit
  int32_t rotate;            // 1: an (s, h)'s partition groups in an order rotated by sh
};

struct FusedArgs {
  StreamArgs st;
  const int32_t* seq_lens;  // int32 [S]
  uint16_t* out;            // bf16 [S][Hkv*QG][128]
  int32_t len_cap;
  int32_t splits;           // workgroups per (s, h), >= 1
  int32_t rotate;           // 1: an (s, h)'s workgroups in an order rotated by sh
  // Cross-workgroup merge workspace, used when splits > 1.
  int32_t* counters;        // [S*Hkv] arrival counters: 0 on entry, re-armed to 0
  float* ws_o;              // [S*Hkv][splits][QG][128] workgroup partials
  float* ws_m;              // [S*Hkv][splits][QG]
  float* ws_l;              // [S*Hkv][splits][QG]
};

// Workgroups per (s, h) of the per-(s, h) fused plan at most.
constexpr int kFusedMaxSplits = 16;

// How the fused kernel is launched: waves per workgroup and workgroups per (s, h).
struct FusedPlan {
  int waves;
  int splits;
};

// A workspace holds the arrival counters first (4 B per (s, h), rounded up to
// 256 B: counter_bytes), then the partials.  `counters` > 0 in the functions
// below gives the counters a fixed region of that many bytes instead (the
// library's static scratch, shared by calls of any size, so that one call's
// partials never land on another call's counters).
size_t counter_bytes(int64_t seq_heads);
// Plan for these sizes with `ws_bytes` of workspace (0: none), and the
// workspace bytes a plan needs (counters first, at a fixed offset).
FusedPlan plan_fused(int64_t seq_heads, int max_seq_len, int query_group_size, size_t ws_bytes,
                     size_t counters = 0, int cus = kFlatGroupsMax);
size_t fused_partial_bytes(int64_t seq_heads, int splits, int query_group_size);
size_t fused_workspace_bytes(int64_t seq_heads, int splits, int query_group_size);
// Carve the workspace for `splits` into the pointers of `a`.
void bind_fused_workspace(FusedArgs* a, void* ws, int64_t seq_heads, int query_group_size,
                          size_t counters = 0);

// Fused decode over one flat work list (the live 32-token chunks of every (s, h)
// in (s, h, chunk) order) dealt evenly to the waves of n_groups
// workgroups of 8 waves.
struct FlatArgs {
  StreamArgs st;
  const int32_t* seq_lens;  // int32 [S]
  uint16_t* out;            // bf16 [S][Hkv*QG][128]
  int32_t len_cap;
  int32_t num_seqs;
  int32_t n_groups;         // the grid
  int32_t* counters;        // [S*Hkv] arrival counters: 0 on entry, re-armed to 0
  float* ws_o;              // [2*n_groups][QG][128] workgroup partials: slot 2g = workgroup
                            // g's first (s, h), 2g+1 = its last
  float* ws_m;              // [2*n_groups][QG]
  float* ws_l;              // [2*n_groups][QG]
};

// Workgroups of the flat plan for these sizes (0: the flat kernel does not
// apply), the workspace bytes it needs, and the carving of that workspace.
// unit_tokens: the tokens of one list entry (a 32-token chunk for the fused path,
// a partition for the two-kernel path).
// cus: the device's compute units (one resident workgroup of 8 waves each).
int plan_flat_groups(int64_t num_seqs, int num_kv_heads, int max_seq_len,
                     int unit_tokens = kFlatUnitTokens, int cus = kFlatGroupsMax);
// Workgroups of the flat partition kernel (tq_partition_flat_kernel) for
// these sizes, or 0 when the per-partition kernel runs instead.
int plan_partition_flat_groups(int64_t num_seqs, int num_kv_heads, int max_seq_len,
                               int partition_tokens, bool tq4, int cus = kFlatGroupsMax);

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount,
// queried once per device; kFlatGroupsMax if the query fails).
int device_cu_count();
size_t flat_partial_bytes(int n_groups, int query_group_size);
size_t flat_workspace_bytes(int64_t seq_heads, int n_groups, int query_group_size);
void bind_flat_workspace(FlatArgs* a, void* ws, int64_t seq_heads, int query_group_size,
                         size_t counters = 0);

// The library's static scratch for tq_decode_fused_static: kStaticScratchBytes
// of device memory per GPU, the first kStaticCounterBytes of them the arrival
// counters.  static_scratch() returns this device's copy (the address comes
// from hipGetSymbolAddress on the first call on each device, which also
// enqueues its zero fill on `stream`).
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr size_t kStaticCounterBytes = size_t(1) << 20;
hipError_t static_scratch(void** ptr, hipStream_t stream);

struct ReduceArgs {
  const float* o;
  const float* ml;
  const float* es;
  const int32_t* seq_lens;
  uint16_t* out;  // bf16 [S][Hkv*QG][128]
  int32_t num_kv_heads;
  int32_t query_group_size;
  int32_t num_partitions;
  int32_t partition_tokens;
  int32_t len_cap;
};

struct KvWriteArgs {
  const uint16_t* k_new;        // bf16 [T][Hkv][128]
  const uint16_t* v_new;        // bf16 [T][Hkv][128]
  const int32_t* slot_mapping;  // [T]: block * BS + offset, negative = skip
  uint8_t* k;                   // e4m3fn, NB blocks of Hkv*BS rows of 128 bytes
  uint8_t* v;
  float* scales;                // fp32 [NB][Hkv][2][BS]
  int32_t row_head_stride;      // as in StreamArgs
  int32_t row_slot_stride;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t kv_block_size;
  int32_t num_slots;            // NB * BS: slots at or past it are skipped
};

// The debug check run before a decode when TQ_VALIDATE=1: one wave per
// sequence reports, by device printf, a length outside [0, max_seq_len] and
// the first block-table entry for t < L outside [0, num_blocks).
struct ValidateArgs {
  const int32_t* bt;        // int32 [S][max_blocks]
  const int32_t* seq_lens;  // int32 [S]
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t kv_block_size;
  int32_t max_seq_len;
};

// Whether the partition kernel stores the partials with the non-temporal bit:
// for fp8 when their bytes (bounded by S * Hkv * P * QG * 520) are large.
bool partials_nontemporal(int64_t num_seqs, int num_kv_heads, int num_partitions,
                          int query_group_size, bool tq4);

// Partitions of one (s, h) that one wave of the partition kernel walks.
int choose_parts_per_wave(int64_t units, int num_partitions);

// Whether the per-unit kernels deal an (s, h)'s workgroups in an order rotated
// by sh: when `waves` exceed one resident round of two waves per SIMD.
bool rotate_units(int64_t waves, int cus);

// Enqueue the kernels; each returns the launch status (hipGetLastError after
// the launch).  launch_partition chooses parts_per_wave and launch_fused the
// waves per workgroup from the sizes.
// tq4 selects the 4-bit record format.
hipError_t launch_partition(PartitionArgs a, int num_seqs, int query_group_size,
                            int kv_block_size, bool tq4, hipStream_t stream);
hipError_t launch_fused(const FusedArgs& a, int num_seqs, int waves, int query_group_size,
                        int kv_block_size, bool tq4, hipStream_t stream);
hipError_t launch_flat(const FlatArgs& a, int query_group_size, int kv_block_size, bool tq4,
                       hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int num_seq_heads, hipStream_t stream);
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_validate(const ValidateArgs& a, hipStream_t stream);

}  // namespace tq
