// Internal interface between the host API and the HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

// Device error word values (match dash_status in include/dash.h).
constexpr int kErrTimeout = -6;
constexpr int kErrPlacement = -7;

struct PreParams {
  const __bf16* o;
  const __bf16* dO;
  float* delta;        // [rows] D = rowsum(dO * O)
  int64_t rows;        // B * H * N
  int* sem;            // ordering semaphores to clear
  int64_t sem_count;
  int* ctr;            // XCD slot counters to clear
  int64_t ctr_count;
  float* dqacc_zero;   // non-null: clear this fp32 buffer (atomic variant)
  int64_t zero_count;  // elements, multiple of 4
};

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;
  const float* lse;
  const float* delta;
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  float* dqacc;
  int* sem;
  int* ctr;
  int* err;
  const int* worker_begin;
  const int4* items;
  const int4* tasks;
  int B, H, Hkv, N;
  int sem_stride;      // semaphores per (b, h), padded
  float scale;         // softmax scale s
  float scale_log2;    // s * log2(e)
  int causal;
  int deterministic;
  int xcd_local;       // 1: every dQ tile's contributors share one XCD (L2)
  int num_xcd;
  int cus_per_xcd;
  long long timeout_ticks;  // wall-clock ticks before a wait gives up
};

hipError_t launch_main(const BwdParams& prm, int d, int nw, int grid, hipStream_t stream);
hipError_t launch_preprocess(const PreParams& prm, int d, int grid, hipStream_t stream);
hipError_t launch_dq_cast(const float* acc, void* dq, int64_t count, float scale, int grid, hipStream_t stream);
hipError_t launch_topology_probe(int* out, int grid, hipStream_t stream);
int main_kernel_lds_bytes(int d, int nw);

}  // namespace dash
