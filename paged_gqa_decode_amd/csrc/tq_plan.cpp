// Host-side planning of the decode launches: how the work is split over
// waves and workgroups, and the workspace layouts of the fused paths.  Host
// code only (no device code, no HIP calls), so it builds with any C++
// compiler; the launchers in tq_kernels.hip use these plans.
#include <stddef.h>
#include <stdint.h>

#include "tq_internal.h"

namespace tq {

namespace {
constexpr int D = kHeadDim;
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

int choose_parts_per_wave(int64_t units, int num_partitions) {
  // Keep enough waves for many rounds over every SIMD; past that, longer
  // per-wave streams amortize each wave's start-up (length, block-table and
  // first-chunk loads, one after the other).
  constexpr int64_t kMinWaves = 32768;
  int64_t ppw = units / kMinWaves;
  if (ppw < 1) ppw = 1;
  if (ppw > num_partitions) ppw = num_partitions;
  return (int)ppw;
}

bool rotate_units(int64_t waves, int cus) {
  // Workgroups go to the 8 XCDs round robin by index.  With an (s, h)'s
  // partitions on consecutive workgroups and a partition count divisible by
  // 8, partition p of every (s, h) lands on XCD p % 8, and on ragged batches,
  // whose high partitions are mostly dead, the XCDs of the low partitions get
  // up to 1.5x the work.  Rotating each (s, h)'s order by sh spreads them:
  // measured on the partition kernel, the ragged workload (16384 one-wave
  // workgroups) 149 -> 119.5 us, the bandwidth workload 414.7 -> 411.5 us; the
  // long-context one, whose 2048 partitions are all resident at once, lost 8 %
  // (79.8 -> 86 us), so the rotation is kept for grids beyond one round.
  const int64_t round = (int64_t)2 * kFlatWaves * (cus < 1 ? 1 : cus);
  return waves > round;
}

bool partials_nontemporal(int64_t num_seqs, int num_kv_heads, int num_partitions,
                          int query_group_size, bool tq4) {
  // Measured on the fp8 partition kernel: with 51-136 MB of partials (bound)
  // the non-temporal bit made the kernel 6-10 % faster, and the whole
  // two-kernel step up to 4 % (the merge then reads the partials from HBM
  // instead of the last-level cache); with 17 MB the step was up to 4 %
  // slower.  The 4-bit partition kernel, bound by its arithmetic, gained
  // nothing and its step lost 3-5 %.
  constexpr int64_t kMinBytes = int64_t(24) << 20;
  const int64_t bytes =
      num_seqs * num_kv_heads * num_partitions * (int64_t)query_group_size * (D + 2) * 4;
  return !tq4 && bytes >= kMinBytes;
}

size_t counter_bytes(int64_t seq_heads) { return round256((size_t)seq_heads * 4); }

size_t fused_partial_bytes(int64_t seq_heads, int splits, int query_group_size) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)seq_heads * splits * query_group_size;
  return round256(rows * D * 4) + 2 * round256(rows * 4);
}

size_t fused_workspace_bytes(int64_t seq_heads, int splits, int query_group_size) {
  if (splits <= 1) return 0;
  return counter_bytes(seq_heads) + fused_partial_bytes(seq_heads, splits, query_group_size);
}

void bind_fused_workspace(FusedArgs* a, void* ws, int64_t seq_heads, int query_group_size,
                          size_t counters) {
  const size_t rows = (size_t)seq_heads * a->splits * query_group_size;
  uint8_t* p = static_cast<uint8_t*>(ws);
  a->counters = reinterpret_cast<int32_t*>(p);
  p += counters ? counters : counter_bytes(seq_heads);
  a->ws_o = reinterpret_cast<float*>(p);
  p += round256(rows * D * 4);
  a->ws_m = reinterpret_cast<float*>(p);
  p += round256(rows * 4);
  a->ws_l = reinterpret_cast<float*>(p);
}

FusedPlan plan_fused(int64_t seq_heads, int max_seq_len, int query_group_size, size_t ws_bytes,
                     size_t counters, int cus) {
  // About 8 waves per CU on the device (one resident round at two waves per
  // SIMD; measured best across the workloads), each with at least one tile
  // group of work; at most 8 waves per workgroup (the register budget of
  // __launch_bounds__(512)), then more workgroups per (s, h) if the workspace
  // can hold their partials.
  const int64_t kTargetWaves = (int64_t)kFlatWaves * (cus < 1 ? 1 : cus);
  const int64_t n_tg = max_seq_len > 0 ? (max_seq_len + kTokensPerTileGroup - 1) / kTokensPerTileGroup : 1;
  int64_t waves_per_sh = (kTargetWaves + seq_heads - 1) / seq_heads;
  if (waves_per_sh > n_tg) waves_per_sh = n_tg;
  if (waves_per_sh < 1) waves_per_sh = 1;
  FusedPlan plan;
  plan.waves = (int)(waves_per_sh < 8 ? waves_per_sh : 8);
  int64_t splits = (waves_per_sh + plan.waves - 1) / plan.waves;
  if (splits > kFusedMaxSplits) splits = kFusedMaxSplits;
  // The counters take their fixed region (counters > 0) or the first bytes the sizes need.
  const size_t cb = counters ? counters : counter_bytes(seq_heads);
  while (splits > 1 && (cb < counter_bytes(seq_heads) ||
                        cb + fused_partial_bytes(seq_heads, (int)splits, query_group_size) > ws_bytes))
    --splits;
  plan.splits = (int)splits;
  return plan;
}

int plan_flat_groups(int64_t num_seqs, int num_kv_heads, int max_seq_len, int unit_tokens,
                     int cus) {
  // One resident round at two waves per SIMD (a workgroup of 8 waves per CU,
  // at most kFlatGroupsMax), or fewer when the list cannot fill them: at most
  // one wave per list entry.
  static_assert(int64_t(kFlatGroupsMax) * kFlatWaves <= 65536, "waves per launch");
  const int64_t kFlatGroups = cus < 1 ? 1 : (cus < kFlatGroupsMax ? cus : kFlatGroupsMax);
  if (num_seqs < 1 || num_seqs > kFlatMaxSeqs || num_kv_heads < 1 || max_seq_len <= 0 ||
      unit_tokens < 1)
    return 0;
  const int64_t n_units = (max_seq_len + unit_tokens - 1) / unit_tokens;
  const int64_t t_max = num_seqs * num_kv_heads * n_units;
  if (t_max > (int64_t(1) << 30)) return 0;
  const int64_t groups = (t_max + kFlatWaves - 1) / kFlatWaves;
  return (int)(groups < kFlatGroups ? groups : kFlatGroups);
}

int plan_partition_flat_groups(int64_t num_seqs, int num_kv_heads, int max_seq_len,
                               int partition_tokens, bool tq4, int cus) {
  // The 4-bit format only, and only when the partitions (bounded by the
  // longest length) fill the resident round: measured faster than one wave per
  // partition there (7-12 % with two rounds of partitions or more, 3 % on the
  // two-kernel step with one round, where its per-lane centroid table spares
  // the bank conflicts of the one-wave workgroups' table).  With fewer
  // partitions than waves its workgroups would leave CUs idle.  No faster for
  // fp8.
  if (!tq4 || num_seqs < 1 || num_kv_heads < 1 || max_seq_len <= 0 || partition_tokens < 1) return 0;
  const int64_t parts = (max_seq_len + partition_tokens - 1) / partition_tokens;
  const int64_t groups = cus < 1 ? 1 : (cus < kFlatGroupsMax ? cus : kFlatGroupsMax);
  if (num_seqs * num_kv_heads * parts < kFlatWaves * groups) return 0;
  return plan_flat_groups(num_seqs, num_kv_heads, max_seq_len, partition_tokens, cus);
}

size_t flat_partial_bytes(int n_groups, int query_group_size) {
  const size_t rows = (size_t)2 * n_groups * query_group_size;
  return round256(rows * D * 4) + 2 * round256(rows * 4);
}

size_t flat_workspace_bytes(int64_t seq_heads, int n_groups, int query_group_size) {
  return counter_bytes(seq_heads) + flat_partial_bytes(n_groups, query_group_size);
}

void bind_flat_workspace(FlatArgs* a, void* ws, int64_t seq_heads, int query_group_size,
                         size_t counters) {
  const size_t rows = (size_t)2 * a->n_groups * query_group_size;
  uint8_t* p = static_cast<uint8_t*>(ws);
  a->counters = reinterpret_cast<int32_t*>(p);
  p += counters ? counters : counter_bytes(seq_heads);
  a->ws_o = reinterpret_cast<float*>(p);
  p += round256(rows * D * 4);
  a->ws_m = reinterpret_cast<float*>(p);
  p += round256(rows * 4);
  a->ws_l = reinterpret_cast<float*>(p);
}

}  // namespace tq
