// What the launcher stand-ins of launch_stubs.cpp recorded.
#pragma once
#include <stddef.h>

struct LaunchLog {
  int partition = 0, fused = 0, flat = 0, reduce = 0, kv_write = 0, validate = 0, scratch = 0;
  bool last_tq4 = false;
  const void* ws = nullptr;  // the workspace the driver passed, to check the carving
  size_t ws_bytes = 0;
  int cus = 256;  // what the device_cu_count stand-in reports
  int flat_partition_groups = -1;  // the flat partition kernel's grid of the last partition launch (0: none)
};
extern LaunchLog g_log;
