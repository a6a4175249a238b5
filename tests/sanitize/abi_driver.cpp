// Drives every entry point of the C ABI, built for the host only with the
// launchers replaced by the recording stand-ins of launch_stubs.cpp, so that
// the argument checks, the size arithmetic and the workspace planning run
// under the address and undefined-behaviour sanitizers.  Device pointers are
// fake aligned addresses (the host code never dereferences them); the fused
// workspace is real host memory, so its carving is checked against the size
// the library asked for.  Exits 0 when every expectation holds.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "launch_log.h"
#include "tq_decode.h"

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    fprintf(stderr, "abi_driver:%d: %s\n", line, what);
    ++g_failures;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void* fake(uintptr_t i) { return reinterpret_cast<void*>(uintptr_t(0x10000000) + 4096 * i); }

struct Case {
  int S, Hkv, QG, BS, G, P, maxlen, NB, mb;
  int layout = TQ_KV_LAYOUT_HEAD_MAJOR;
};

tq_extent extent(const Case& c) {
  tq_extent e;
  e.num_seqs = c.S;
  e.num_blocks = c.NB;
  e.max_blocks_per_seq = c.mb;
  e.num_partitions = c.P;
  e.max_seq_len = c.maxlen;
  e.head_dim = 128;
  e.kv_layout = c.layout;
  return e;
}

void run_valid(const Case& c) {
  const tq_extent e = extent(c);
  const float scale = 0.088388f;
  tq_partials part = {(float*)fake(10), (float*)fake(11), (float*)fake(12)};
  EXPECT(tq_partials_bytes(&e, c.Hkv, c.QG) > 0);
  const LaunchLog before = g_log;
  EXPECT(tq_decode(fake(1), (const uint8_t*)fake(2), (const uint8_t*)fake(3), (const float*)fake(4),
                   (const int32_t*)fake(5), (const int32_t*)fake(6), &part, c.Hkv, c.QG, c.BS, c.G,
                   scale, &e, nullptr) == TQ_OK);
  EXPECT(g_log.partition == before.partition + 1 && !g_log.last_tq4);
  EXPECT(tq_decode_reduce(&part, (const int32_t*)fake(6), fake(7), c.Hkv, c.QG, c.G, &e,
                          nullptr) == TQ_OK);
  EXPECT(g_log.reduce == before.reduce + 1);
  EXPECT(tq4_decode(fake(1), (const uint8_t*)fake(2), (const float*)fake(4), (const int32_t*)fake(5),
                    (const int32_t*)fake(6), &part, c.Hkv, c.QG, c.BS, c.G, scale, &e,
                    nullptr) == TQ_OK);
  EXPECT(g_log.partition == before.partition + 2 && g_log.last_tq4);

  // Fused: without a workspace, then with exactly the bytes the library asks for.
  for (int fmt = 0; fmt < 2; ++fmt) {
    const size_t ws_bytes = tq_fused_workspace_bytes(&e, c.Hkv, c.QG);
    std::vector<uint8_t> ws(ws_bytes + 256);
    uint8_t* wsp = ws.data() + ((256 - ((uintptr_t)ws.data() & 255)) & 255);
    for (int with_ws = 0; with_ws < 2; ++with_ws) {
      void* w = with_ws && ws_bytes ? wsp : nullptr;
      g_log.ws = w;
      g_log.ws_bytes = w ? ws_bytes : 0;
      const int launches = g_log.fused + g_log.flat;
      const tq_status st =
          fmt == 0 ? tq_decode_fused(fake(1), (const uint8_t*)fake(2), (const uint8_t*)fake(3),
                                     (const float*)fake(4), (const int32_t*)fake(5),
                                     (const int32_t*)fake(6), fake(7), c.Hkv, c.QG, c.BS, c.G,
                                     scale, &e, w, g_log.ws_bytes, nullptr)
                   : tq4_decode_fused(fake(1), (const uint8_t*)fake(2), (const float*)fake(4),
                                      (const int32_t*)fake(5), (const int32_t*)fake(6), fake(7),
                                      c.Hkv, c.QG, c.BS, c.G, scale, &e, w, g_log.ws_bytes,
                                      nullptr);
      EXPECT(st == TQ_OK);
      EXPECT(g_log.fused + g_log.flat == launches + 1);
      EXPECT(g_log.last_tq4 == (fmt == 1));
      g_log.ws = nullptr;
    }
  }
  // The entry point that allocates nothing: the static scratch (host memory in the stand-in).
  {
    const int launches = g_log.fused + g_log.flat;
    EXPECT(tq_decode_fused_static(fake(1), (const uint8_t*)fake(2), (const uint8_t*)fake(3),
                                  (const float*)fake(4), (const int32_t*)fake(5),
                                  (const int32_t*)fake(6), fake(7), c.Hkv, c.QG, c.BS, c.G, scale,
                                  &e, nullptr) == TQ_OK);
    EXPECT(g_log.fused + g_log.flat == launches + 1);
    g_log.ws = nullptr;
  }
}

// Which partition kernel the two-kernel path plans: the flat one for the 4-bit
// format once the partitions (bounded by max_seq_len) fill one resident round of
// 8 waves per CU, one wave per partition otherwise and always for fp8.
void run_partition_plans() {
  struct PlanCase {
    Case c;
    int cus;
    bool flat;
  };
  const PlanCase cases[] = {
      {{16, 4, 16, 32, 5, 32, 40960, 14336, 1280}, 256, true},   // 2048 partitions: one round
      {{16, 4, 16, 32, 5, 32, 40959, 14336, 1280}, 256, true},   // still 32 partitions each
      {{16, 4, 16, 32, 5, 32, 39680, 14336, 1280}, 256, false},  // 31 each: 1984 < 2048
      {{1, 4, 16, 32, 5, 32, 40960, 1280, 1280}, 256, false},    // one sequence
      {{1, 4, 16, 32, 5, 32, 40960, 1280, 1280}, 16, true},      // ... on a 16-CU device
      {{128, 8, 8, 32, 1, 32, 8192, 32768, 256}, 256, true},
  };
  for (const PlanCase& pc : cases) {
    g_log.cus = pc.cus;
    const tq_extent e = extent(pc.c);
    tq_partials part = {(float*)fake(10), (float*)fake(11), (float*)fake(12)};
    EXPECT(tq4_decode(fake(1), (const uint8_t*)fake(2), (const float*)fake(4),
                      (const int32_t*)fake(5), (const int32_t*)fake(6), &part, pc.c.Hkv, pc.c.QG,
                      pc.c.BS, pc.c.G, 0.088f, &e, nullptr) == TQ_OK);
    EXPECT((g_log.flat_partition_groups > 0) == pc.flat);
    EXPECT(g_log.flat_partition_groups <= pc.cus);
    EXPECT(tq_decode(fake(1), (const uint8_t*)fake(2), (const uint8_t*)fake(3), (const float*)fake(4),
                     (const int32_t*)fake(5), (const int32_t*)fake(6), &part, pc.c.Hkv, pc.c.QG,
                     pc.c.BS, pc.c.G, 0.088f, &e, nullptr) == TQ_OK);
    EXPECT(g_log.flat_partition_groups == 0);
  }
  g_log.cus = 256;
}

void run_static_limits() {
  // More (sequence, kv head) pairs than the static counter region holds: refused, no launch.
  const Case c = {1024, 257, 8, 16, 1, 2, 300, 64, 32};
  const tq_extent e = extent(c);
  const LaunchLog before = g_log;
  EXPECT(tq_decode_fused_static(fake(1), (const uint8_t*)fake(2), (const uint8_t*)fake(3),
                                (const float*)fake(4), (const int32_t*)fake(5),
                                (const int32_t*)fake(6), fake(7), c.Hkv, c.QG, c.BS, c.G, 0.088f,
                                &e, nullptr) == TQ_ERR_SCRATCH);
  EXPECT(g_log.fused == before.fused && g_log.flat == before.flat && g_log.scratch == before.scratch);
}

void run_invalid() {
  const Case c = {4, 2, 8, 16, 1, 2, 300, 64, 32};
  tq_extent e = extent(c);
  tq_partials part = {(float*)fake(10), (float*)fake(11), (float*)fake(12)};
  auto dec = [&](const tq_extent* ep, int Hkv, int QG, int BS, int G, float sc, const void* q) {
    return tq_decode(q, (const uint8_t*)fake(2), (const uint8_t*)fake(3), (const float*)fake(4),
                     (const int32_t*)fake(5), (const int32_t*)fake(6), &part, Hkv, QG, BS, G, sc,
                     ep, nullptr);
  };
  const LaunchLog before = g_log;
  EXPECT(dec(&e, 2, 8, 16, 1, 0.1f, nullptr) == TQ_ERR_NULL);
  EXPECT(dec(nullptr, 2, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_NULL);
  EXPECT(dec(&e, 2, 7, 16, 1, 0.1f, fake(1)) == TQ_ERR_UNSUPPORTED);
  EXPECT(dec(&e, 2, 8, 64, 1, 0.1f, fake(1)) == TQ_ERR_UNSUPPORTED);
  EXPECT(dec(&e, 0, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_SHAPE);
  EXPECT(dec(&e, 2, 8, 16, 0, 0.1f, fake(1)) == TQ_ERR_SHAPE);
  EXPECT(dec(&e, 2, 8, 16, 1, 0.f, fake(1)) == TQ_ERR_SCALE);
  EXPECT(dec(&e, 2, 8, 16, 1, -1.f, fake(1)) == TQ_ERR_SCALE);
  EXPECT(dec(&e, 2, 8, 16, 1, 1.f / 0.f, fake(1)) == TQ_ERR_SCALE);
  EXPECT(dec(&e, 2, 8, 16, 1, 0.1f, (const char*)fake(1) + 2) == TQ_ERR_MISALIGNED);
  e.max_seq_len = 2 * 256 + 1;  // past P * E
  EXPECT(dec(&e, 2, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_COVERAGE);
  e.max_seq_len = -1;
  EXPECT(dec(&e, 2, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_COVERAGE);
  e = extent(c);
  e.head_dim = 64;
  EXPECT(dec(&e, 2, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_UNSUPPORTED);
  e = extent(c);
  // sizes whose products overflow 32-bit indices
  e.num_seqs = 1 << 20;
  e.num_partitions = 1 << 12;
  EXPECT(dec(&e, 1024, 8, 16, 1, 0.1f, fake(1)) == TQ_ERR_SHAPE);
  e = extent(c);
  EXPECT(dec(&e, 2, 8, 16, (1 << 30), 0.1f, fake(1)) == TQ_ERR_SHAPE);
  EXPECT(g_log.partition == before.partition);  // nothing launched

  // the writer
  auto kvw = [&](int T, int Hkv, int BS, int NB, int hd, const void* kn, int layout = 0) {
    return tq_kv_write(kn, fake(21), (const int32_t*)fake(22), (uint8_t*)fake(23),
                       (uint8_t*)fake(24), (float*)fake(25), T, Hkv, BS, NB, hd, layout, nullptr);
  };
  EXPECT(kvw(4, 2, 16, 8, 128, fake(20), 2) == TQ_ERR_UNSUPPORTED);
  EXPECT(kvw(0, 2, 16, 8, 128, nullptr) == TQ_OK);
  EXPECT(kvw(4, 2, 16, 8, 128, nullptr) == TQ_ERR_NULL);
  EXPECT(kvw(4, 2, 24, 8, 128, fake(20)) == TQ_ERR_UNSUPPORTED);
  EXPECT(kvw(4, 2, 16, 8, 64, fake(20)) == TQ_ERR_UNSUPPORTED);
  EXPECT(kvw(-1, 2, 16, 8, 128, fake(20)) == TQ_ERR_SHAPE);
  EXPECT(kvw(1 << 30, 4, 16, 8, 128, fake(20)) == TQ_ERR_SHAPE);
  EXPECT(kvw(4, 2, 16, 1 << 30, 128, fake(20)) == TQ_ERR_SHAPE);
  EXPECT(kvw(4, 2, 16, 8, 128, (const char*)fake(20) + 4) == TQ_ERR_MISALIGNED);
  EXPECT(g_log.kv_write == before.kv_write);
  EXPECT(kvw(4, 2, 16, 8, 128, fake(20)) == TQ_OK);
  EXPECT(g_log.kv_write == before.kv_write + 1);
  EXPECT(kvw(4, 2, 16, 8, 128, fake(20), TQ_KV_LAYOUT_SLOT_MAJOR) == TQ_OK);
  EXPECT(g_log.kv_write == before.kv_write + 2);

  // sizes of the 4-bit record, status strings, version
  EXPECT(tq4_block_bytes(8, 32) == (size_t)8 * 32 * 134);
  EXPECT(tq4_block_bytes(8, 24) == 0);
  EXPECT(tq4_block_bytes(0, 32) == 0);
  for (int s = 0; s < 9; ++s) EXPECT(strlen(tq_status_str((tq_status)s)) > 0);
  EXPECT(strcmp(tq_status_str((tq_status)99), "unknown status") == 0);
  EXPECT(tq_abi_version() == TQ_ABI_VERSION);
  EXPECT(tq_last_hip_error() == 0);
}

}  // namespace

int main() {
  const Case valid[] = {
      {1, 1, 8, 16, 1, 1, 256, 16, 16},           // one partition
      {32, 8, 8, 16, 1, 16, 4096, 8192, 256},     // uniform batch
      {64, 8, 6, 32, 1, 32, 8192, 9216, 256},     // ragged batch
      {128, 8, 8, 32, 1, 32, 8192, 32768, 256},   // the bandwidth workload
      {16, 4, 16, 32, 5, 32, 40960, 14336, 1280}, // long contexts, G = 5
      {300, 2, 16, 16, 2, 4, 2000, 4000, 128},    // more sequences than the flat plan takes
      {3, 1, 6, 32, 1, 4, 0, 4, 4},               // every length 0
      {1, 1, 8, 32, 4096, 1, 1 << 20, 40000, 1 << 15},  // one very long sequence
  };
  for (const Case& c : valid) run_valid(c);
  for (Case c : valid) {  // the page's slot-major row order
    c.layout = TQ_KV_LAYOUT_SLOT_MAJOR;
    run_valid(c);
  }
  for (int cus : {32, 80, 304}) {  // devices of other sizes (partitioned modes, larger parts)
    g_log.cus = cus;
    for (const Case& c : valid) run_valid(c);
  }
  g_log.cus = 256;
  run_partition_plans();
  run_invalid();
  run_static_limits();
  setenv("TQ_VALIDATE", "1", 1);
  const int v0 = g_log.validate;
  run_valid(valid[1]);
  EXPECT(g_log.validate > v0);
  unsetenv("TQ_VALIDATE");
  if (g_failures) {
    fprintf(stderr, "abi_driver: %d expectation(s) failed\n", g_failures);
    return 1;
  }
  printf("abi_driver: all expectations hold (%d partition, %d fused, %d flat, %d reduce, %d writer, %d validate launches)\n",
         g_log.partition, g_log.fused, g_log.flat, g_log.reduce, g_log.kv_write, g_log.validate);
  return 0;
}
