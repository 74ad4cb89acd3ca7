// Device-side helpers shared by the HIP kernels of the attention backward (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dash {


typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (round to nearest even) in one dword, a in the low half.
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const floatx2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))
#define CONST_AS __attribute__((address_space(4)))

// One record of the schedule table (item or task), read field by field through the
// constant address space.
struct Quad {
  int x, y, z, w;
};
__device__ __forceinline__ Quad load_quad(const CONST_AS Quad* tab, int i) {
  const CONST_AS int* f = reinterpret_cast<const CONST_AS int*>(tab + i);
  return Quad{f[0], f[1], f[2], f[3]};
}

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// MFMAs written as inline assembly, for operands or accumulators held in AGPRs (the
// compiler's MFMA form is one register file per function). The compiler's hazard checks
// do not look inside inline assembly: an MFMA must not read a VGPR that a VALU
// instruction wrote less than 2 wait states before it. The S/dP and dQ MFMAs
// (mfma32_vab*) read only LDS loads and AGPRs, so they carry no wait; the dV/dK MFMAs
// read the packed P and dS, which the compiler may convert right before their first use,
// so they start with s_nop 1. tests/test_asm_hazards.py checks the compiled kernels for
// every violation. Back-to-back MFMAs accumulating into the same registers need no
// wait states; reads of a VGPR result by other instructions need mfma_result_wait().
//
// dK/dV accumulation with the accumulator pinned in AGPRs: these 32x32 fp32 blocks are
// touched only by MFMAs for a whole KV item, so keeping them out of the VGPRs leaves
// the VGPRs to the softmax and to operands in flight. Dependent MFMAs on the same
// accumulator are at least 7 MFMAs apart here.
__device__ __forceinline__ void mfma32_acc(floatx16& acc, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Accumulator in VGPRs, B operand in AGPRs (an operand held for a whole KV item).
__device__ __forceinline__ void mfma32_vab(floatx16& acc, bf16x8 a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// Moves an operand that only AGPR-operand MFMAs read into AGPRs once, so that the
// register allocator keeps it there (instead of a VGPR copy moved over per use).
__device__ __forceinline__ bf16x8 to_agpr(bf16x8 v) {
  asm volatile("" : "+a"(v));
  return v;
}
// The same starting from a zero accumulator.
__device__ __forceinline__ void mfma32_vab_zero(floatx16& acc, bf16x8 a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
// Wait states between an inline-assembly MFMA writing `acc` (VGPRs) and memory or VALU
// instructions reading it (12 for a store, 13 for VALU; 16 given). Ties the value to
// the wait so that no reader is scheduled before it.
__device__ __forceinline__ void mfma_result_wait(floatx16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc));
}
__device__ __forceinline__ void mfma_result_wait(floatx16& x, floatx16& y) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
// Wait states between MFMAs writing AGPR accumulators and any other reader of them
// (v_accvgpr_read, stores): 13, more than an 8-pass MFMA needs. The accumulators are tied
// to the wait, so that no read of them is scheduled before it.
__device__ __forceinline__ void mfma_settle(floatx16 (&a)[2], floatx16 (&b)[2]) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[0]), "+a"(a[1]), "+a"(b[0]), "+a"(b[1]));
}
__device__ __forceinline__ void mfma_settle(floatx16 (&a)[2]) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[0]), "+a"(a[1]));
}
__device__ __forceinline__ void mfma_settle(floatx16 (&a)[4]) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
__device__ __forceinline__ void mfma_settle(floatx16 (&a)[4], floatx16 (&b)[4]) {
  asm volatile("s_nop 7\n\ts_nop 4"
               : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(b[0]), "+a"(b[1]), "+a"(b[2]), "+a"(b[3]));
}

// Scheduling hints (__builtin_amdgcn_sched_group_barrier): the instructions of the
// current scheduling region are placed in groups of `n` instructions of a class, in
// the order the calls appear.
enum SchedClass { kSchedVALU = 0x2, kSchedMFMA = 0x8, kSchedDSRead = 0x100, kSchedDSWrite = 0x200 };
#define SCHED_GROUP(cls, n) __builtin_amdgcn_sched_group_barrier((cls), (n), 0)

__device__ __forceinline__ unsigned xcc_id() {
  // HW_REG_XCC_ID (hwreg 20), bits [3:0]: the XCD this wave runs on.
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xfu;
}

__device__ __forceinline__ int load_flag_sys(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void raise_error(int* err, int code) {
  // The operands are made here (an empty asm hides them from the compiler), so that it
  // does not keep them live from the kernel's start for this rarely taken path.
  int expected = 0;
  asm volatile("" : "+v"(expected), "+v"(code));
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8) that waits for LDS and scalar-memory operations only: lgkmcnt(0).
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt immediate that waits until at most n (0..63) vector-memory operations of
// this wave are outstanding: vmcnt(n).
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Waits until every memory operation this wave issued has completed: global stores
// acknowledged by the L2, global->LDS copies landed. The signal fences keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void wait_mem_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Spin (the whole wave, one shared address) until *sem == want. Returns false if the
// wait timed out or another wave reported an error; the caller then skips its
// reduction step but keeps going, so that every barrier is still reached and the
// kernel drains. Semaphores are read with agent-scope loads, which skip the CU's L1
// and see the latest device-scope store from any XCD. No fence follows: the data the
// turn guards must itself be read with device-scope loads when the writer may sit on
// another XCD (whose L2 is not coherent with this one's).
__device__ bool wait_turn(const int* sem, int want, int* err, long long timeout_ticks) {
  const long long t0 = wall_clock64();
  int iter = 0;
  while (true) {
    const int s = __builtin_amdgcn_readfirstlane(__hip_atomic_load(sem, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (s == want) break;
    if ((++iter & 31) == 0) {
      if (__builtin_amdgcn_readfirstlane(load_flag_sys(err)) != 0) return false;
      if (wall_clock64() - t0 > timeout_ticks) {
        if (__lane_id() == 0) raise_error(err, kErrTimeout);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return true;
}

// Profiling builds (-DDASH_PROFILE) accumulate per-wave cycle counts (s_memtime) of
// the phases of a step; see ProfSlot. Other builds compile the marks away.
#ifdef DASH_PROFILE
#define PROF_DECL                                      \
  unsigned long long prof_acc[kProfSlots] = {};        \
  unsigned long long prof_t = __builtin_readcyclecounter(); \
  const unsigned long long prof_t0 = prof_t;
#define PROF_MARK(slot)                                            \
  do {                                                             \
    const unsigned long long prof_now = __builtin_readcyclecounter(); \
    prof_acc[slot] += prof_now - prof_t;                           \
    prof_t = prof_now;                                             \
  } while (0)
#define PROF_COUNT(slot) (prof_acc[slot] += 1)
#define PROF_STORE(prm, wave, nw)                                                       \
  do {                                                                                  \
    if ((prm).prof && (threadIdx.x & 63) == 0) {                                        \
      prof_acc[kProfTotal] = __builtin_readcyclecounter() - prof_t0;                     \
      unsigned long long* dst = (prm).prof + (static_cast<size_t>(blockIdx.x) * (nw) + (wave)) * kProfSlots; \
      for (int k_ = 0; k_ < kProfSlots; ++k_) dst[k_] = prof_acc[k_];                    \
    }                                                                                   \
  } while (0)
#else
#define PROF_DECL
#define PROF_MARK(slot) ((void)0)
#define PROF_COUNT(slot) ((void)0)
#define PROF_STORE(prm, wave, nw) ((void)0)
#endif

// Semaphore read through the scalar unit, bypassing the scalar cache (glc): served by
// the L2 and counted by lgkmcnt, so polling does not wait for the vector-memory queue
// (global->LDS copies in flight).
__device__ __forceinline__ int sload_glc(const int* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Wave-level wait for the dQ turn (XCD-local chains): scalar polls of *sem until it
// equals `want`. Returns false on timeout or when another wave reported an error.
__device__ bool wait_turn_local(const int* sem, int want, int* err, long long timeout_ticks) {
  if (sload_glc(sem) == want) return true;
  const long long t0 = wall_clock64();
  int iter = 0;
  while (true) {
    __builtin_amdgcn_s_sleep(1);
    if (sload_glc(sem) == want) return true;
    if ((++iter & 31) == 0) {
      if (sload_glc(err) != 0) return false;
      if (wall_clock64() - t0 > timeout_ticks) {
        if (__lane_id() == 0) raise_error(err, kErrTimeout);
        return false;
      }
    }
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end return 0 and
// stores past the end are dropped, which is how rows past N are skipped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Buffer cache policies. SC0 alone: the load misses the CU's L1 and reads the XCD's L2,
// the coherence point of CUs on one XCD. SC1: device scope, past the XCD's L2 (needed
// when writer and reader may sit on different XCDs).
constexpr int kSC0 = 1;
constexpr int kSC1 = 16;
// (The raw buffer load/store builtins move 32-bit patterns as unsigned int: float
// data is bit-cast, never converted.)

// ---------------------------------------------------------------------------------
// LDS tiles. Tiles are row-major bf16 with one 16-byte pad chunk per row (row stride
// = row bytes + 16), so that consecutive rows start 16 bytes apart modulo the 256
// bytes the 64 LDS banks cover.
//
// Row permutation. The 32 rows m of an MFMA operand (lane % 32) read Q/dO rows
// pi(m), where pi swaps the two 2-bit fields of m inside each aligned group of 16:
// m = 16G + 4a + j -> pi(m) = 16G + a + 4j. Then
//  - the sixteen lanes of one ds_read_b128 phase read sixteen different rows, i.e.
//    sixteen different 16-byte bank groups (conflict-free), and
//  - four consecutive accumulator rows m..m+3 (what one ds_read_b64_tr_b16 group
//    gathers for the P^T dO and dS^T Q operands) are physical rows four apart, so a
//    transpose read of 4 rows x 4 chunks also hits sixteen different bank groups.
// The same trick orders the KV rows of the dQ = dS K contraction (its k index):
// k-step kk, lane half hi, read s and group row j use KV row 16kk + 2hi + s + 4j,
// for both operands.
// Every LDS address is then "per-lane part + compile-time constant".
// ---------------------------------------------------------------------------------
template <int D>
struct TileGeom {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int STRIDE = 2 * D + 16;   // bytes per LDS row
};
constexpr int kDsStride = 128 + 16;  // dS^T tile [kv][64 q]: bytes per LDS row

__device__ __forceinline__ int pi16(int m) { return (m & ~15) | ((m >> 2) & 3) | ((m & 3) << 2); }

__device__ __forceinline__ bf16x8 lds_ld16(const LDS_AS char* base, int off) {
  return *reinterpret_cast<const LDS_AS bf16x8*>(base + off);
}

// Transpose read (ds_read_b64_tr_b16): lane j of each 16-lane group receives column
// (n0 + j) of the group's 4 rows; this lane supplies the address of its row and of
// the 4 columns n0 + 4*(lane%4) .. +3 (byte offset `off`).
__device__ __forceinline__ shortx4 lds_tr(const LDS_AS char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<LDS_AS shortx4*>(const_cast<LDS_AS char*>(base) + off));
}

__device__ __forceinline__ bf16x8 join(shortx4 a, shortx4 b) {
  typedef short shortx8 __attribute__((ext_vector_type(8)));
  const shortx8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Global -> LDS copies (global_load_lds, scalar base + 32-bit per-lane byte offset):
// lane l's bytes land at lds_base + l * size. They are issued through inline assembly
// so that the compiler does not treat them as LDS stores: otherwise it waits for them
// (s_waitcnt vmcnt(0)) before every LDS read of the other buffer. Their completion is
// awaited explicitly (wait_mem_done) before the barrier that publishes the buffer.
__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, LDS_AS char* lds_base) {
  const unsigned m0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds_base));
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* sbase, unsigned voff, LDS_AS char* lds_base) {
  const unsigned m0 = static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds_base));
  asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Copy plan of a ROWS x D bf16 tile into a padded LDS tile: instruction m of wave w
// fills LDS slots [64 blk, 64 blk + 64), blk = w + NW m; lane l's slot holds chunk c
// of row r. voff[m] is the lane's byte offset (r D + 8 c) * 2 from the tile's first
// global row (pad slots re-read chunk 0 of their row: harmless). Computed once.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int SPR = TileGeom<D>::CPR + 1;  // slots per row
  static constexpr int NI = ROWS * SPR / 64;         // instructions per tile
  static constexpr int PER_WAVE = (NI + NW - 1) / NW;
  static_assert((ROWS * SPR) % 64 == 0, "tile must fill whole 1 KiB blocks");
  unsigned voff[PER_WAVE];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int m = 0; m < PER_WAVE; ++m) {
      const int slot = (w + NW * m) * 64 + lane;
      const int r = slot / SPR;
      int c = slot - r * SPR;
      c = c < TileGeom<D>::CPR ? c : 0;
      voff[m] = static_cast<unsigned>((r * D + c * 8) * 2);
    }
  }
  // Rows [r0, r0 + ROWS) of the row-major [nrows, D] matrix at src (0 <= r0, 1 <= nrows;
  // r0 may be >= nrows for a step past the end). Rows past nrows repeat row nrows - 1
  // (finite values; the kernel masks them): then every offset is taken from row 0 of
  // the matrix with the row clamped in signed arithmetic, so no address leaves
  // [src, src + nrows * D).
  // Instruction m (< PER_WAVE) of this wave's share of the copy below, alone; issues
  // nothing where the wave has no block m.
  __device__ __forceinline__ void issue_one(LDS_AS char* dst, const bf16* src, int r0, int nrows, int w, int m) const {
    if (!(m + 1 < PER_WAVE || w + NW * m < NI)) return;
    if (r0 + ROWS <= nrows) {
      dma16(src + static_cast<int64_t>(r0) * D, voff[m], dst + (w + NW * m) * 1024);
    } else {
      int r = r0 + static_cast<int>(voff[m] / (2 * D));
      r = r < nrows - 1 ? r : nrows - 1;
      dma16(src, static_cast<unsigned>(r) * (2 * D) + (voff[m] % (2 * D)), dst + (w + NW * m) * 1024);
    }
  }
  // The same without a branch on raggedness: the clamped addressing above always (three
  // VALU instructions per copy).
  __device__ __forceinline__ void issue_one_clamped(LDS_AS char* dst, const bf16* src, int r0, int nrows, int w,
                                                    int m) const {
    if (!(m + 1 < PER_WAVE || w + NW * m < NI)) return;
    int r = r0 + static_cast<int>(voff[m] / (2 * D));
    r = r < nrows - 1 ? r : nrows - 1;
    dma16(src, static_cast<unsigned>(r) * (2 * D) + (voff[m] % (2 * D)), dst + (w + NW * m) * 1024);
  }
  __device__ __forceinline__ void issue(LDS_AS char* dst, const bf16* src, int r0, int nrows, int w) const {
    if (r0 + ROWS <= nrows) {  // wave-uniform: whole tile inside the matrix
      const bf16* base = src + static_cast<int64_t>(r0) * D;
#pragma unroll
      for (int m = 0; m < PER_WAVE; ++m) {
        // Blocks of the first PER_WAVE - 1 rounds always exist: NW (PER_WAVE - 1) < NI.
        if (m + 1 < PER_WAVE || w + NW * m < NI) dma16(base, voff[m], dst + (w + NW * m) * 1024);
      }
    } else {
#pragma unroll
      for (int m = 0; m < PER_WAVE; ++m) {
        if (m + 1 < PER_WAVE || w + NW * m < NI) {
          int r = r0 + static_cast<int>(voff[m] / (2 * D));
          r = r < nrows - 1 ? r : nrows - 1;
          const unsigned v = static_cast<unsigned>(r) * (2 * D) + (voff[m] % (2 * D));
          dma16(src, v, dst + (w + NW * m) * 1024);
        }
      }
    }
  }
};

// 64 floats of rows r0 + pi(m) (clamped to < nrows) into LDS slot m, one dword per lane.
// As in TileCopy::issue, a ragged step addresses from row 0 with a signed clamp.
__device__ __forceinline__ void dma_row64(LDS_AS char* dst, const float* src, int r0, int nrows, int lane) {
  if (r0 + 64 > nrows) {
    int r = r0 + pi16(lane);
    r = r < nrows - 1 ? r : nrows - 1;
    dma4(src, static_cast<unsigned>(r * 4), dst);
  } else {
    dma4(src + r0, static_cast<unsigned>(pi16(lane) * 4), dst);
  }
}

}  // namespace dash
