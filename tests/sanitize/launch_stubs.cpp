// Stand-ins for the kernel launchers of tq_kernels.hip, for a host-only build
// of the C ABI (tq_api.cpp + tq_plan.cpp) under the address and
// undefined-behaviour sanitizers: each records the launch and checks the
// arguments that the host code prepared, and launches nothing.
#include <stdio.h>
#include <stdlib.h>

#include "launch_log.h"
#include "tq_internal.h"

LaunchLog g_log;

namespace {
void require(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "launch stub: %s\n", what);
    abort();
  }
}
// The row strides of either order: one of them is a single 128-byte row.
void require_row_strides(int head_stride, int slot_stride, int Hkv, int BS) {
  require((head_stride == BS * 128 && slot_stride == 128) ||
              (head_stride == 128 && slot_stride == Hkv * 128),
          "row strides");
}
bool in_range(const void* p, const void* base, size_t bytes) {
  return (const char*)p >= (const char*)base && (const char*)p <= (const char*)base + bytes;
}
}  // namespace

namespace tq {

hipError_t launch_partition(PartitionArgs a, int num_seqs, int query_group_size, int kv_block_size,
                            bool tq4, hipStream_t) {
  ++g_log.partition;
  require(num_seqs >= 1 && a.num_partitions >= 1 && a.partition_tokens >= 256, "partition sizes");
  require(query_group_size == 6 || query_group_size == 8 || query_group_size == 16, "QG");
  require(kv_block_size == 16 || kv_block_size == 32, "BS");
  require(a.o && a.ml && a.es && a.seq_lens && a.st.bt && a.st.q, "partition pointers");
  require_row_strides(a.st.row_head_stride, a.st.row_slot_stride, a.st.num_kv_heads, kv_block_size);
  require(tq4 ? (a.st.tq4 && a.st.centroids) : (a.st.k && a.st.v && a.st.scales), "format");
  // The launcher's plan: the flat kernel's grid, else one wave per run of partitions.
  const int flat_groups = plan_partition_flat_groups(num_seqs, a.st.num_kv_heads, a.len_cap,
                                                     a.partition_tokens, tq4, g_log.cus);
  require(flat_groups >= 0 && flat_groups <= 256 && (tq4 || flat_groups == 0), "flat partition plan");
  g_log.flat_partition_groups = flat_groups;
  const bool nt = partials_nontemporal(num_seqs, a.st.num_kv_heads, a.num_partitions,
                                       query_group_size, tq4);
  require(!(nt && tq4), "partial store policy");
  if (flat_groups == 0) {
    const int ppw = choose_parts_per_wave((int64_t)num_seqs * a.st.num_kv_heads * a.num_partitions,
                                          a.num_partitions);
    require(ppw >= 1 && ppw <= a.num_partitions, "parts per wave");
  }
  g_log.last_tq4 = tq4;
  return hipSuccess;
}

hipError_t launch_fused(const FusedArgs& a, int num_seqs, int waves, int query_group_size,
                        int kv_block_size, bool tq4, hipStream_t) {
  ++g_log.fused;
  require(num_seqs >= 1 && waves >= 1 && waves <= 8 && a.splits >= 1, "fused plan");
  require(a.splits == 1 || (a.counters && a.ws_o && a.ws_m && a.ws_l), "fused workspace");
  require(query_group_size >= 1 && kv_block_size >= 1, "fused sizes");
  if (a.splits > 1 && g_log.ws) {
    require(in_range(a.ws_l, g_log.ws, g_log.ws_bytes), "fused workspace carving");
  }
  g_log.last_tq4 = tq4;
  return hipSuccess;
}

hipError_t launch_flat(const FlatArgs& a, int query_group_size, int kv_block_size, bool tq4,
                       hipStream_t) {
  ++g_log.flat;
  require(a.n_groups >= 1 && a.n_groups <= 256 && a.n_groups <= g_log.cus && a.num_seqs >= 1,
          "flat plan");
  require(a.counters && a.ws_o && a.ws_m && a.ws_l, "flat workspace");
  require(query_group_size >= 1 && kv_block_size >= 1, "flat sizes");
  if (g_log.ws) {
    // the last carved array ends inside the workspace the caller passed
    const size_t rows = (size_t)2 * a.n_groups * query_group_size;
    require(in_range(a.ws_l + rows, g_log.ws, g_log.ws_bytes), "flat workspace carving");
  }
  g_log.last_tq4 = tq4;
  return hipSuccess;
}

hipError_t launch_reduce(const ReduceArgs& a, int num_seq_heads, hipStream_t) {
  ++g_log.reduce;
  require(num_seq_heads >= 1 && a.num_partitions >= 1 && a.o && a.out, "reduce args");
  return hipSuccess;
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t) {
  ++g_log.kv_write;
  require(a.num_tokens >= 1 && a.num_kv_heads >= 1 && a.num_slots >= 1, "writer args");
  require_row_strides(a.row_head_stride, a.row_slot_stride, a.num_kv_heads, a.kv_block_size);
  return hipSuccess;
}

int device_cu_count() { return g_log.cus; }

// The static scratch of tq_decode_fused_static: real host memory of the same size, recorded
// as the workspace so that the launch stand-ins check the carving against it.
hipError_t static_scratch(void** ptr, hipStream_t) {
  static uint8_t* mem = static_cast<uint8_t*>(aligned_alloc(256, kStaticScratchBytes));
  require(mem != nullptr, "scratch stand-in");
  ++g_log.scratch;
  g_log.ws = mem;
  g_log.ws_bytes = kStaticScratchBytes;
  *ptr = mem;
  return hipSuccess;
}

hipError_t launch_validate(const ValidateArgs& a, hipStream_t) {
  ++g_log.validate;
  require(a.num_seqs >= 1 && a.bt && a.seq_lens, "validate args");
  return hipSuccess;
}

}  // namespace tq
