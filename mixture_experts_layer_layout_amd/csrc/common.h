// common.h -- shared device helpers for the gfx950 MoE kernels: element
// conversions, MFMA wrappers, bounded device-side waits and signals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_PROTO_FN __host__ __device__ __forceinline__
#include "protocol.h"
#include "slots.h"

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;  // every kernel runs 4 waves of 64

// ---------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

typedef __bf16 bf16x2_hw_t __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest even: the conversion compiles to the
// gfx950 instruction v_cvt_pk_bf16_f32 (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Two floats as packed bfloat16 (lo in bits 0-15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_hw_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// A pointer that is the same in every lane of the wave, moved to scalar
// registers (the compiler cannot prove it uniform when it derives from
// values loaded from memory).
__device__ __forceinline__ void* wave_uniform(void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// Buffer descriptor for raw (untyped) buffer accesses from base: no stride,
// 2^31 - 1 bytes in range, word 3 = 32-bit data format as gfx9-family
// parts expect for raw buffer instructions.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}

// The value of the neighbouring lane (lane ^ 1) through a DPP quad
// permutation [1,0,3,2] (one VALU instruction, no LDS round trip).
__device__ __forceinline__ float swap_lane_pair(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------- MFMA
// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).  Each lane supplies 8
// consecutive-k values of one A row and of one B column; lanes 0-31 and
// 32-63 cover the two halves of k.  Output register r of lane l holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- waits
// Producer -> consumer hand-off between workgroups, possibly on different
// XCDs (each XCD has its own, non-coherent L2):
//   producer  every wave waits for its stores to reach the L2, then one
//             wave writes the XCD's L2 back (agent-scope release) and bumps
//             the counter
//   consumer  thread 0 polls the counter with relaxed agent-scope atomic
//             loads (coherent, no cache maintenance) and the workgroup
//             proceeds behind a workgroup-scope acquire
// The consumer invalidates no cache, so no L1 or L2 may hold a copy of the
// data it reads that is older than the producer's stores.  That holds when
// every 128-byte line of an exchanged buffer has one producer task in a
// launch and is read in that launch only by tasks that waited for that
// producer: a line read earlier could only have been brought in by a reader
// of other data on the same line.  So every buffer exchanged inside a launch
// is laid out with each producer's bytes in lines of their own (row-tile
// slots of 128-byte multiples, 128-byte aligned row strides and slice
// strides), and the dispatch's own acquire leaves no copy from earlier
// launches.  (An agent-scope acquire would invalidate the XCD's whole L2 at
// every wait, destroying the reuse of the operand rows other workgroups
// share there.)  The one exchanged array whose lines have several
// producers is inv (each token's k slots, written by the gather tasks of
// the row tiles the token went to); a reader in the same launch (the merge
// under MOE_FLAG_PERSISTENT_SINGLE) loads it with coherent agent-scope
// loads instead.  The router's logit slices (and the top-k's indices,
// gates and mask bytes) are stored coherently and published by
// signal_add_stored: published by the write-back, the top-k
// on another XCD now and then read 256 bytes of a slice before the
// router's values reached it (with a workspace pre-filled with a byte
// pattern, some builds showed the pattern's logits for 2 or 4 tokens in up
// to 38 of 270 calls; with the coherent stores none in 684).
// The claim and wait logic itself is protocol.h, shared with a host model.
struct DevOps {
  static __device__ __forceinline__ int load(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ __forceinline__ int fetch_add(int* p, int v) { return atomicAdd(p, v); }
  static __device__ __forceinline__ void store(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ __forceinline__ void set_status(int32_t* s, int c) {
    if (s) atomicCAS((int*)s, 0, c);
  }
  static __device__ __forceinline__ void pause() { __builtin_amdgcn_s_sleep(2); }
};

using proto::WaitCtx;

__device__ __forceinline__ int load_relaxed(const int* p) { return DevOps::load(p); }

__device__ __forceinline__ void set_status(int32_t* status, int code) { DevOps::set_status(status, code); }

// Thread 0 only: true when *ctr >= target; false on timeout/abort.
__device__ __forceinline__ bool thread_wait_geq(const int* ctr, int target, const WaitCtx& w) {
  return proto::wait_geq<DevOps>(ctr, target, w);
}

// Block-uniform: true when *ctr >= target; false on timeout/abort.
__device__ __forceinline__ bool wait_geq(const int* ctr, int target, const WaitCtx& w, int* lds_flag) {
  if (threadIdx.x == 0) *lds_flag = thread_wait_geq(ctr, target, w) ? 1 : 0;
  __syncthreads();
  const int ok = *lds_flag;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  __syncthreads();
  return ok != 0;
}

// Block-uniform: publishes every prior global store of the workgroup at
// agent scope, then adds `v` to *ctr.  The agent-scope release writes the
// XCD's L2 back, which is costly; REL = false skips it and is correct only
// when every reader of the published data runs in a later kernel launch
// (the end of a kernel writes the L2s back and the next launch starts with
// an acquire).  The count itself is still raised, atomically at agent scope.
template <bool REL = true>
__device__ __forceinline__ void signal_add(int* ctr, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (REL) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Cache policy of a store written through the XCD's L2 to memory, coherent
// at agent scope (the sc1 bit, as the compiler sets it on agent-scope atomic
// stores): a workgroup on another XCD that has not cached the line reads
// the stored value from memory.
constexpr int kStoreCoherent = 16;

// Block-uniform: adds `v` to *ctr once every wave's earlier stores have
// completed.  For data stored coherently (kStoreCoherent) this publishes it
// to readers in the same launch without writing any L2 back: each wave waits
// for its stores (s_waitcnt vmcnt(0): a coherent store completes once it is
// performed in memory), the barrier orders the waves, and the count follows.
__device__ __forceinline__ void signal_add_stored(int* ctr, int v) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters untouched
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait states after a store of more than 8 bytes, before anything else
// issues.  Such a store reads its data registers after it has issued, and
// the compiler may put an instruction that overwrites them right behind it
// (the register holding a stored word, reused for the next accumulator
// tile or an address).  On gfx950 that was seen to change what was stored:
// now and then, in some lanes, the first word of a 16-byte store held the
// value written by the next instruction (zeros, address bits).  Every
// 16-byte store issued through a builtin here is followed by this guard;
// a host test checks the built kernels for the pattern.
__device__ __forceinline__ void store_data_guard() {
  __builtin_amdgcn_sched_barrier(0);  // nothing moves between the store and the wait
  asm volatile("s_nop 3");
  __builtin_amdgcn_sched_barrier(0);
}

// 16 bytes stored coherently (kStoreCoherent) at byte offset `off` of a
// buffer whose base is the same in every lane.
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t rs, int off, uint4 v) {
  typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
  u32x4_t q;
  q[0] = v.x; q[1] = v.y; q[2] = v.z; q[3] = v.w;
  __builtin_amdgcn_raw_buffer_store_b128(q, rs, off, 0, kStoreCoherent);
  store_data_guard();
}
__device__ __forceinline__ void store_coherent_u8(__amdgpu_buffer_rsrc_t rs, int off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, rs, off, 0, kStoreCoherent);
}

// ---------------------------------------------------------------- copies
// One wave copies one row of nvec 16-byte vectors: every lane issues up to
// kCopyUnroll loads before its first store (the source and destination may
// alias as far as the compiler knows, so a plain loop would wait for each
// load in turn).  f(v, u) may transform each vector before it is stored.
constexpr int kCopyUnroll = 16;  // a whole d = 7168 bf16 row (14 vectors a lane) in one batch
template <class F>
__device__ __forceinline__ void wave_copy_row(const uint4* __restrict__ src, uint4* __restrict__ dst, int nvec,
                                              F f) {
  const int lane = threadIdx.x & 63;
  for (int v0 = lane; v0 < nvec; v0 += 64 * kCopyUnroll) {
    uint4 t[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (v0 + 64 * u < nvec) t[u] = src[v0 + 64 * u];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (v0 + 64 * u < nvec) dst[v0 + 64 * u] = f(v0 + 64 * u, t[u]);
  }
}

struct CopyAsIs {
  __device__ __forceinline__ uint4 operator()(int, uint4 u) const { return u; }
};

// One wave writes one source row to k <= 64 destination rows, reading it
// once: every lane loads up to kCopyUnroll vectors, then stores them to each
// destination.  Lane j holds destination j's row index in lane_row (read
// out with readlane, so no memory load sits between the stores: vmcnt
// counts stores too, and a load there would wait for every store before
// it); indices outside [0, R) are skipped.  f(j, u) may transform a vector
// for destination j.
template <class F>
__device__ __forceinline__ void wave_push_row(const uint4* __restrict__ src, uint4* __restrict__ dst, int nvec,
                                              int k, int R, int lane_row, F f) {
  const int lane = threadIdx.x & 63;
  for (int v0 = lane; v0 < nvec; v0 += 64 * kCopyUnroll) {
    uint4 u[kCopyUnroll];
#pragma unroll
    for (int q = 0; q < kCopyUnroll; ++q)
      if (v0 + 64 * q < nvec) u[q] = src[v0 + 64 * q];
    for (int j = 0; j < k; ++j) {
      const int r = __builtin_amdgcn_readlane(lane_row, j);
      if ((unsigned)r >= (unsigned)R) continue;
      uint4* d = dst + (size_t)r * nvec;
#pragma unroll
      for (int q = 0; q < kCopyUnroll; ++q)
        if (v0 + 64 * q < nvec) d[v0 + 64 * q] = f(j, u[q]);
    }
  }
}

// ---------------------------------------------------------------- misc
__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace moe
