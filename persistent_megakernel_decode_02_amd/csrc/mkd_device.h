// Device code of the persistent decode megakernel for gfx950 (MI355X): one
// sequence (dense or MoE model) or 2-8 sequences decoded together (dense),
// each its own instantiation of the same persistent loop (one translation
// unit per kernel: mkd_kernel_dense.hip, mkd_kernel_moe.hip,
// mkd_kernel_batch.hip; the launch code is in mkd_launch.hip).
//
// One cooperative launch; one 512-thread workgroup per compute unit; every
// workgroup walks its slice of a host-built instruction tensor for every
// decode step and never exits early (Kittens VM summary, "Method";
// Hyperkernel teardown, "What a megakernel buys").
//
// Synchronisation.  Instead of a separate counter per stage, every value an
// instruction produces is published as one 64-bit word {fp32 value, 32-bit
// tag}, stored with an agent-scope atomic store; the tag is the dependency
// counter of that (step, layer) and a consumer spins on the words it needs
// until each carries the expected tag.  A 64-bit store is single-copy atomic,
// so a word with the right tag holds the right value; no release fence or
// counter round trip sits between a producer's last store and its consumers'
// first useful load.  The pages' principle of removing fences between
// pipeline stages (epic-kernel README, "Fence removal and barrier reduction")
// taken to its end on a device whose L2 is split across 8 XCDs.
//
// Weight streaming.  Batch-1 GEMV is one multiply-add per weight, far below
// the MFMA ridge point, so no matrix cores: each wavefront streams whole rows
// with coalesced 16-byte (dwordx4) non-temporal loads into a ring of
// registers, RING loads deep per lane (64 KiB per CU in flight), and issues
// an instruction's first RING loads *before* waiting on its inputs, so weight
// traffic overlaps the dependency wait (epic-kernel README, "Pipelining for
// B200 bandwidth" and "L2 prefetching overlapped with prior instructions";
// Hyperkernel teardown: next-layer tiles load while the current layer runs).
// Wavefront reductions use DPP row permutes plus readlane.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "mkd_internal.h"

namespace mkd {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Explicit address spaces: pointers read from the weight table carry none, and
// generic (flat) accesses would make the compiler wait for every outstanding
// memory operation, serialising the weight stream.
#define GLOBAL __attribute__((address_space(1)))
typedef GLOBAL const u32x4 g_u32x4;

__device__ __forceinline__ u32x4 ld_nt16(const void* p) {
  return __builtin_nontemporal_load((g_u32x4*)p);
}
__device__ __forceinline__ uint16_t ld_u16(const void* p) { return *(GLOBAL const uint16_t*)p; }
__device__ __forceinline__ float ld_f32(const void* p) { return *(GLOBAL const float*)p; }
__device__ __forceinline__ int ld_i32(const void* p) { return *(GLOBAL const int*)p; }
__device__ __forceinline__ uint64_t ld_u64(const void* p) { return *(GLOBAL const uint64_t*)p; }
// Tables that stay constant for a whole launch (weight pointers, the
// instruction tensor) are read through the constant address space: uniform
// addresses then become scalar loads and the values live in scalar registers.
#define CONSTANT __attribute__((address_space(4)))
__device__ __forceinline__ uint64_t ldc_u64(const void* p) { return *(CONSTANT const uint64_t*)p; }
__device__ __forceinline__ int ldc_i32(const void* p) { return *(CONSTANT const int*)p; }

// The launch parameters, read in place from the kernel-argument segment.
// Keeping the constant address space on every access matters: a load
// through a generic pointer counts as divergent (generic addresses may be
// per-lane scratch), which would move every pointer and loop bound derived
// from the parameters into vector registers.
typedef CONSTANT const KParams CKParams;
__device__ __forceinline__ void st_f32(float* p, float v) { *(GLOBAL float*)p = v; }
__device__ __forceinline__ void st_i32(int32_t* p, int32_t v) { *(GLOBAL int32_t*)p = v; }
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) { *(GLOBAL uint64_t*)p = v; }

constexpr int RING = 8;       // 16-byte weight loads in flight per lane (GEMV)
constexpr int ARING = 4;      // K/V position steps in flight per lane (attention)
constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer descriptor word 3 (gfx9 family)
constexpr int kSC1 = 16;                     // cache-policy bit: device-coherent access
constexpr int kNT = 2;                       // cache-policy bit: non-temporal (streamed once)

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf_val(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// fp32 -> bf16, round to nearest even (values here are finite)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// LDS words shared by the workgroup's wavefronts.  The explicit address
// space matters: a volatile access through a generic pointer becomes a flat
// load, which also counts against the vector-memory counter, so the wait for
// it would wait for every weight load in flight.
typedef __attribute__((address_space(3))) volatile int lds_vint;
__device__ __forceinline__ void ll_store(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float lane_read(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// sum over each group of 8 lanes, result in all 8 lanes
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  return v;
}
// sum over each row of 16 lanes, result in all 16 lanes
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
// sum over the wavefront, wave-uniform result
__device__ __forceinline__ float wave_sum(float v) {
  v = sum16(v);
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// Wavefront sums of four values at once.  Two values trade half-waves
// (v_permlane32_swap) and are added, so one register holds the 32-lane
// partial sums of both (lanes 0-31 the first, 32-63 the second); two such
// registers trade 16-lane rows (v_permlane16_swap) and are added, so each
// row holds the 16-lane partials of one value; a row reduction finishes.
// Row r of the result holds the sum of v[kQuadValue[r]] in all its lanes.
// (10 instructions for four sums, against 11 per sum with wave_sum.)
constexpr int kQuadValue[4] = {0, 2, 1, 3};
__device__ __forceinline__ float quad_sum(float v0, float v1, float v2, float v3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
  const float u01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float u23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u01), __float_as_uint(u23), false, false);
  return sum16(__uint_as_float(c[0]) + __uint_as_float(c[1]));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufFlags);
}

// a if !b else c, as integer selects (keeps pointer choices out of memory)
__device__ __forceinline__ const uint16_t* psel(bool b, const uint16_t* x, const uint16_t* y) {
  const uint64_t m = 0ull - (uint64_t)b;
  return (const uint16_t*)(((uint64_t)x & ~m) | ((uint64_t)y & m));
}

__device__ __forceinline__ uint32_t tag_of(CKParams& p, int t, int l) {
  return 1u + (uint32_t)t * (uint32_t)(p.L + 1) + (uint32_t)l;
}

__device__ __forceinline__ const uint16_t* wptr(CKParams& p, int slot) {
  return (const uint16_t*)ldc_u64(p.wtab + slot);
}
__device__ __forceinline__ const uint16_t* lptr(CKParams& p, int layer, int slot) {
  return (const uint16_t*)ldc_u64(p.wtab + W_GLOBAL + layer * p.lslots + slot);
}

// ---------------------------------------------------------------- per-workgroup context

struct Ctx {
  CKParams& p;
  float* xs;     // staged input vector   [x_floats]
  float* res;    // residual rows         [res_floats]
  float* out;    // GEMV row results      [out_floats]
  float* red;    // reduction scratch     [kRed]
  lds_vint* sflag;  // LDS ints: [0] abort, [1] token, [2] token step, [3..6] route
  int wg, instr, t, tid, lane, wave;
  int stage, index;                              // from the instruction words
  uint64_t* tr;                                  // this instruction's trace entry, or null
  int seq;                                       // sequence of a per-sequence instruction
  int B;                                         // sequences decoded together (a constant 1
                                                 // in the batch-1 kernel)
};

// Record a device error: the first raiser records where; with stop_all every
// other workgroup's waits end too.
__device__ __forceinline__ void raise_at(int32_t* status, lds_vint* sflag, int code, bool stop_all,
                                         int wg, int instr, int t) {
  int expected = 0;
  if (__hip_atomic_compare_exchange_strong(&status[S_CODE], &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(&status[S_WG], wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&status[S_INSTR], instr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&status[S_TOKEN], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (stop_all) {
    __hip_atomic_store(&status[S_ABORT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sflag[0] = 1;
  }
}

__device__ __forceinline__ void raise_error(Ctx& c, int code, bool stop_all) {
  raise_at(c.p.status, c.sflag, code, stop_all, c.wg, c.instr, c.t);
}

// Staging tagged words into LDS.  A fetch reads the 16-byte aligned span
// that covers src[0..n) -- every activation buffer is a whole number of
// 128-byte lines, so the span stays inside it -- two tagged words per
// 16-byte load, S loads per thread in flight per batch (loads past the span
// read zeros: the descriptor covers exactly the span).  Words whose tag is
// still old are then polled one by one, with backoff, until they are
// current, the launch is aborted (stop word, another workgroup's error) or
// the watchdog deadline passes.  No barrier: callers end with sync_ok().
struct Span {
  const uint64_t* w0;  // first word of the aligned span
  int lead;            // words of the span before src (0 or 1)
  int npairs;          // 16-byte loads covering the span
};

__device__ __forceinline__ Span span_of(const uint64_t* src, int n) {
  Span sp;
  const uintptr_t s0 = (uintptr_t)src & ~(uintptr_t)15;
  sp.w0 = (const uint64_t*)s0;
  sp.lead = (int)(((uintptr_t)src - s0) >> 3);
  sp.npairs = n > 0 ? (sp.lead + n + 1) >> 1 : 0;
  return sp;
}

template <int S>
struct Staged {
  u32x4 v[S];
};

template <int S>
__device__ __forceinline__ void ll_issue(Ctx& c, const Span& sp, int base, Staged<S>& st) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(sp.w0, (uint32_t)sp.npairs * 16u);
#pragma unroll
  for (int k = 0; k < S; ++k)
    st.v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (base + k * kThreads + c.tid) * 16, 0, kSC1);
}

// Where word i of a fetch lands in its LDS destination: in place, or (input
// vectors of several sequences) in 8 NB-word slices padded by 4 words (SlicePad).
struct InPlace {
  __device__ __forceinline__ int operator()(int i) const { return i; }
};
// The input vectors of NB sequences, interleaved (element k of sequence b is
// word k NB + b), are read by the batched GEMV one 8-element slice per lane:
// 8 NB consecutive floats.  Unpadded, lane l's slice starts at 32 NB l bytes,
// so 16 consecutive lanes fall on as few as one 16-byte bank group of LDS
// (NB = 8) and every slice read is serialised.  Each slice is followed by 4
// padding floats: lane l then starts at bank group (2 NB + 1) l mod 16, odd
// times l, which is a different group for each of 16 consecutive lanes.
template <int NB>
struct SlicePad {
  static constexpr int kStride = 8 * NB + 4;  // floats from one slice to the next
  __device__ __forceinline__ int operator()(int i) const { return i + (i / (8 * NB)) * 4; }
};

// A thread's words still to come are two bits per 16-byte load k of a batch
// (bit 2k: the pair's first word, bit 2k + 1: its second) of a 32-bit mask,
// so a batch has at most 16 loads per thread: a shift by 32 or more is
// undefined, and the compiler may then drop words that are still pending.
template <int S, class M = InPlace>
__device__ __forceinline__ void ll_finish(Ctx& c, const Span& sp, int base, const Staged<S>& st, int n,
                                          uint32_t tag, float* dst, M m = M()) {
  static_assert(S >= 1 && S <= 16, "two pending bits per load in a 32-bit mask");
  unsigned pending = 0;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int i0 = 2 * (base + k * kThreads + c.tid) - sp.lead;
    if (i0 >= 0 && i0 < n) {
      if (st.v[k].y == tag) dst[m(i0)] = __uint_as_float(st.v[k].x);
      else pending |= 1u << (2 * k);
    }
    if (i0 + 1 >= 0 && i0 + 1 < n) {
      if (st.v[k].w == tag) dst[m(i0 + 1)] = __uint_as_float(st.v[k].z);
      else pending |= 2u << (2 * k);
    }
  }
  if (!pending) return;
  // some producer's store is still in flight: re-read the pairs that hold
  // such words, all of them in one round trip, until every word is current
  const uint64_t t0 = wall_clock64();
  const __amdgpu_buffer_rsrc_t r = make_rsrc(sp.w0, (uint32_t)sp.npairs * 16u);
  for (int it = 0; pending; ++it) {
    __builtin_amdgcn_s_sleep(1);
    u32x4 v[S];
#pragma unroll
    for (int k = 0; k < S; ++k)
      if ((pending >> (2 * k)) & 3u)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (base + k * kThreads + c.tid) * 16, 0, kSC1);
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int i0 = 2 * (base + k * kThreads + c.tid) - sp.lead;
      if ((pending & (1u << (2 * k))) && v[k].y == tag) {
        dst[m(i0)] = __uint_as_float(v[k].x);
        pending &= ~(1u << (2 * k));
      }
      if ((pending & (2u << (2 * k))) && v[k].w == tag) {
        dst[m(i0 + 1)] = __uint_as_float(v[k].z);
        pending &= ~(2u << (2 * k));
      }
    }
    // (the stop word lives in host memory: a read of it crosses PCIe, and
    // every wavefront of the chip re-reading it here queued those reads for
    // hundreds of microseconds; a stop reaches these loops as the abort word,
    // which workgroup 0 raises when its per-step read finds the stop word)
    if (pending && (it & 15) == 15) {
      if (c.sflag[0] ||
          __hip_atomic_load(&c.p.status[S_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        c.sflag[0] = 1;
        break;
      }
      if (wall_clock64() - t0 > c.p.watchdog_ticks) {
        raise_error(c, MKD_E_WATCHDOG, true);
        break;
      }
    }
  }
}

// batches of one fetch from pair `from` on, S loads per thread each
template <int S, class M = InPlace>
__device__ __forceinline__ void ll_fetch_from(Ctx& c, const uint64_t* src, int n, uint32_t tag, float* dst,
                                              int from, M m = M()) {
  const Span sp = span_of(src, n);
  for (int base = from; base < sp.npairs; base += S * kThreads) {
    Staged<S> st;
    ll_issue<S>(c, sp, base, st);
    ll_finish<S, M>(c, sp, base, st, n, tag, dst, m);
  }
}
template <class M = InPlace>
__device__ __forceinline__ void ll_fetch(Ctx& c, const uint64_t* src, int n, uint32_t tag, float* dst, M m = M()) {
  ll_fetch_from<8, M>(c, src, n, tag, dst, 0, m);
}

// workgroup barrier; false when the launch is being aborted
// (values read from LDS after a barrier are the same in every lane; reading
// them through readfirstlane tells the compiler so, which keeps the control
// flow that depends on them uniform and its loop counters in scalar registers)
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ bool sync_ok(Ctx& c) {
  __syncthreads();
  return uni(c.sflag[0]) == 0;
}

// Mark this instruction done for this step: a barrier (the next instruction
// reuses the LDS areas the epilogue read) and the instruction's completion
// flag, step + 1.  No consumer waits on the flags -- inputs are recognised by
// their tags -- they are the launch's progress record: after an abort or a
// watchdog error they show how far each instruction got.
__device__ __forceinline__ void signal_done(Ctx& c) {
  __syncthreads();
  if (c.tid == 0) {
    __hip_atomic_store(c.p.flags + (size_t)c.stage * c.p.flag_stride + c.index, (uint32_t)(c.t + 1),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c.tr) st_u64(c.tr + 2, wall_clock64());
  }
}

__device__ __forceinline__ void mark_ready(Ctx& c) {
  if (c.tr && c.tid == 0) st_u64(c.tr + 1, wall_clock64());
}


// sum of v over the workgroup (all threads call; result in all threads)
__device__ __forceinline__ float block_sum(Ctx& c, float v) {
  v = wave_sum(v);
  if (c.lane == 0) c.red[c.wave] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += c.red[w];
  __syncthreads();
  return s;
}

// One tagged input vector: n words at src, expected tag, LDS destination.
struct Fetch {
  const uint64_t* src;
  int n;
  uint32_t tag;
  float* dst;
};

// Stage an instruction's inputs, with no wait on the producers' flags: every
// thread reads its share of the words at once and re-reads, one round trip
// per round, the pairs whose tag is still old until every word is current.
// Each word is caught as soon as its producer's store lands, instead of a
// round trip after the producing stage's last flag.  (A flag wait first, or
// until at most 64 producers were left, measured slower; re-reading the host
// stop word in these loops is what once made this scheme erratic.)
// The first batch of up to three fetches is issued before any is checked, so
// one round trip covers an instruction's inputs (8192 words of the first,
// 2048 of the others); longer inputs take further batches.
// (the first fetch's words land in its destination through m; S0 16-byte
// loads per thread per batch of it)
template <int K, class M = InPlace, int S0 = 8>
__device__ __forceinline__ bool gather(Ctx& c, const Fetch (&f)[K], M m = M()) {
  constexpr int S1 = 2;
  Staged<S0> st0;
  Staged<S1> st1, st2;
  const Span sp0 = span_of(f[0].src, f[0].n);
  ll_issue<S0>(c, sp0, 0, st0);
  Span sp1{}, sp2{};
  if (K > 1) {
    sp1 = span_of(f[1].src, f[1].n);
    ll_issue<S1>(c, sp1, 0, st1);
  }
  if (K > 2) {
    sp2 = span_of(f[2].src, f[2].n);
    ll_issue<S1>(c, sp2, 0, st2);
  }
  ll_finish<S0, M>(c, sp0, 0, st0, f[0].n, f[0].tag, f[0].dst, m);
  if (K > 1) ll_finish<S1>(c, sp1, 0, st1, f[1].n, f[1].tag, f[1].dst);
  if (K > 2) ll_finish<S1>(c, sp2, 0, st2, f[2].n, f[2].tag, f[2].dst);
  ll_fetch_from<S0, M>(c, f[0].src, f[0].n, f[0].tag, f[0].dst, S0 * kThreads, m);
  if (K > 1) ll_fetch_from<S1>(c, f[1].src, f[1].n, f[1].tag, f[1].dst, S1 * kThreads);
  if (K > 2) ll_fetch_from<S1>(c, f[2].src, f[2].n, f[2].tag, f[2].dst, S1 * kThreads);
#pragma unroll
  for (int j = 3; j < K; ++j) ll_fetch(c, f[j].src, f[j].n, f[j].tag, f[j].dst);
  if (!sync_ok(c)) return false;
  mark_ready(c);
  return true;
}

template <int K, class M = InPlace, int S0 = 8>
__device__ __forceinline__ bool gather_inputs(Ctx& c, const Fetch (&f)[K], M m = M()) {
  return gather<K, M, S0>(c, f, m);
}

// Stage small inputs without waiting for the producing stage's flags: every
// thread re-reads its words (one 16-byte load per pair of words, pairs
// tid, tid + kThreads, ...) until each carries the expected tag.  The
// instruction then waits only for the producers of the words it reads -- an
// attention instruction for the few QKV tiles that hold its head's q, k and
// v rows, a split-KV reduction for its head's chunk partials -- and saves the
// round trip of the flag poll.  Only for inputs of at most kThreads * S word
// pairs read by few instructions: the reads repeat until the data is there.
// The abort word and the deadline are looked at every 32 rounds, by each
// wavefront as a whole (a stop request arrives as the abort word).
template <int S>
__device__ __forceinline__ bool ll_poll(Ctx& c, const uint64_t* src, int n, uint32_t tag, float* dst) {
  CKParams& p = c.p;
  const Span sp = span_of(src, n);
  static_assert(S >= 1 && S <= 16, "two pending bits per load in a 32-bit mask");
  unsigned pending = 0;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const int i0 = 2 * (k * kThreads + c.tid) - sp.lead;
    if (i0 >= 0 && i0 < n) pending |= 1u << (2 * k);
    if (i0 + 1 >= 0 && i0 + 1 < n) pending |= 2u << (2 * k);
  }
  const uint64_t t0 = wall_clock64();
  for (int it = 0;; ++it) {
    Staged<S> st;
    ll_issue<S>(c, sp, 0, st);
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int i0 = 2 * (k * kThreads + c.tid) - sp.lead;
      if ((pending & (1u << (2 * k))) && st.v[k].y == tag) {
        dst[i0] = __uint_as_float(st.v[k].x);
        pending &= ~(1u << (2 * k));
      }
      if ((pending & (2u << (2 * k))) && st.v[k].w == tag) {
        dst[i0 + 1] = __uint_as_float(st.v[k].z);
        pending &= ~(2u << (2 * k));
      }
    }
    if (__builtin_amdgcn_ballot_w64(pending != 0) == 0) return true;   // this wavefront's words are in
    __builtin_amdgcn_s_sleep(1);
    if ((it & 31) == 31) {
      int stop = 0;
      if (c.sflag[0] || __hip_atomic_load(&p.status[S_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        stop = 1;
      } else if (wall_clock64() - t0 > p.watchdog_ticks) {
        stop = 3;
      }
      stop = uni(stop);
      if (stop) {
        if (c.lane == 0) {
          if (stop == 1) c.sflag[0] = 1;
          else raise_error(c, MKD_E_WATCHDOG, true);
        }
        return false;
      }
    }
  }
}

// As ll_poll, for K inputs of at most kThreads word pairs each, polled
// together: per round, one 16-byte load per thread and input, issued only
// while that pair still holds an old word, so one round trip covers all K.
template <int K>
__device__ __forceinline__ bool ll_poll_k(Ctx& c, const Fetch (&f)[K]) {
  CKParams& p = c.p;
  Span sp[K];
  static_assert(K <= 16, "two pending bits per input in a 32-bit mask");
  unsigned pending = 0;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    sp[k] = span_of(f[k].src, f[k].n);
    const int i0 = 2 * c.tid - sp[k].lead;
    if (i0 >= 0 && i0 < f[k].n) pending |= 1u << (2 * k);
    if (i0 + 1 >= 0 && i0 + 1 < f[k].n) pending |= 2u << (2 * k);
  }
  const uint64_t t0 = wall_clock64();
  for (int it = 0;; ++it) {
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
      if ((pending >> (2 * k)) & 3u)
        v[k] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(sp[k].w0, (uint32_t)sp[k].npairs * 16u),
                                                     c.tid * 16, 0, kSC1);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int i0 = 2 * c.tid - sp[k].lead;
      if ((pending & (1u << (2 * k))) && v[k].y == f[k].tag) {
        f[k].dst[i0] = __uint_as_float(v[k].x);
        pending &= ~(1u << (2 * k));
      }
      if ((pending & (2u << (2 * k))) && v[k].w == f[k].tag) {
        f[k].dst[i0 + 1] = __uint_as_float(v[k].z);
        pending &= ~(2u << (2 * k));
      }
    }
    if (__builtin_amdgcn_ballot_w64(pending != 0) == 0) return true;   // this wavefront's words are in
    __builtin_amdgcn_s_sleep(1);
    if ((it & 31) == 31) {
      int stop = 0;
      if (c.sflag[0] || __hip_atomic_load(&p.status[S_ABORT], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        stop = 1;
      } else if (wall_clock64() - t0 > p.watchdog_ticks) {
        stop = 3;
      }
      stop = uni(stop);
      if (stop) {
        if (c.lane == 0) {
          if (stop == 1) c.sflag[0] = 1;
          else raise_error(c, MKD_E_WATCHDOG, true);
        }
        return false;
      }
    }
  }
}

// RMSNorm gains of this thread's elements (i = tid + k * kThreads), read
// before the inputs are waited for; covers d <= kGainRegs * kThreads
constexpr int kGainRegs = 8;
struct Gains {
  float g[kGainRegs];
};
__device__ __forceinline__ Gains load_gains(Ctx& c, int d, const uint16_t* gamma) {
  Gains r;
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = c.tid + k * kThreads;
    r.g[k] = bf_val(ld_u16(gamma + (i < d ? i : d - 1)));
  }
  return r;
}

// xs[0..d) <- rmsnorm(xs) * gamma  (fp32)
__device__ __forceinline__ void rmsnorm_g(Ctx& c, int d, const uint16_t* gamma, const Gains& gr) {
  float ss = 0.f;
  for (int i = c.tid; i < d; i += kThreads) ss = fmaf(c.xs[i], c.xs[i], ss);
  const float tot = block_sum(c, ss);
  const float inv = 1.0f / sqrtf(tot / (float)d + c.p.eps);
#pragma unroll
  for (int k = 0; k < kGainRegs; ++k) {
    const int i = c.tid + k * kThreads;
    if (i < d) c.xs[i] = (c.xs[i] * inv) * gr.g[k];
  }
  for (int i = c.tid + kGainRegs * kThreads; i < d; i += kThreads)
    c.xs[i] = (c.xs[i] * inv) * bf_val(ld_u16(gamma + i));
  __syncthreads();
}

// ---------------------------------------------------------------- token selection

// (value, index) maximum with the lowest index on ties
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// argmax of sequence sq's logits from the LM-head tile partials staged in
// LDS at xs: (max, argmax) pairs in tile order, the sequences interleaved
// (word w of sequence sq at xs[w * B + sq])
__device__ __forceinline__ int argmax_staged(Ctx& c, int sq) {
  CKParams& p = c.p;
  const int B = c.B;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int k = c.tid; k < p.n_lm_tiles; k += kThreads) {
    const float v = c.xs[(2 * k) * B + sq];
    const int i = __float_as_int(c.xs[(2 * k + 1) * B + sq]);
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  int* ired = (int*)(c.red + 64);
  if (c.lane == 0) { c.red[c.wave] = bv; ired[c.wave] = bi; }
  __syncthreads();
  bv = c.red[0];
  bi = ired[0];
  for (int w = 1; w < kWaves; ++w)
    if (better(c.red[w], ired[w], bv, bi)) { bv = c.red[w]; bi = ired[w]; }
  __syncthreads();
  return uni(bi);
}

// every sequence's LM-head tile partials of step tt, staged in LDS at xs
// (re-read until every tile's pair is current)
__device__ __forceinline__ bool fetch_partials(Ctx& c, int tt) {
  CKParams& p = c.p;
  const Fetch f[1] = {{p.lm, 2 * p.n_lm_tiles * c.B, tag_of(p, tt, p.L), c.xs}};
  return gather<1>(c, f);
}

// Every sequence's token of step sflag[2], kept at the end of the reduction
// scratch (words kTokWord .. + kMaxBatch are used by nothing else).  A
// static __shared__ array here instead moved the dynamic LDS area and cost
// 2% of batch-1 decode time.
constexpr int kTokWord = 240;
static_assert(kTokWord + kMaxBatch <= kRed, "token words inside the reduction scratch");
__device__ __forceinline__ int* step_tok(Ctx& c) { return (int*)(c.red + kTokWord); }

// tokens consumed at step t by every sequence, into step_tok (computed once per
// step and workgroup; workgroup 0 records the previous step's argmax)
__device__ __forceinline__ bool step_tokens(Ctx& c) {
  CKParams& p = c.p;
  if (uni(c.sflag[2]) == c.t) return true;
  __syncthreads();  // every thread is done with the previous step's tokens
  if (c.t == 0) {
    if (c.tid == 0)
      for (int b = 0; b < c.B; ++b) step_tok(c)[b] = p.first_tok[b];
  } else {
    // teacher forcing (one sequence): workgroup 0 still folds the argmax to record it
    const int f = p.forced ? uni(ld_i32(p.forced + c.t)) : -1;
    if (f < 0 || c.wg == 0) {
      if (!fetch_partials(c, c.t - 1)) return false;
      for (int b = 0; b < c.B; ++b) {
        const int am = argmax_staged(c, b);
        if (c.tid == 0) {
          if (c.wg == 0) st_i32(p.tokens_out + (size_t)b * p.n_steps + c.t - 1, am);
          if (f < 0) step_tok(c)[b] = am;
        }
      }
    }
    if (f >= 0 && c.tid == 0) step_tok(c)[0] = f;
  }
  __syncthreads();
  bool bad = false;
  for (int b = 0; b < c.B; ++b) bad = bad || step_tok(c)[b] < 0 || step_tok(c)[b] >= p.V;
  if (bad) {
    if (c.tid == 0) raise_error(c, MKD_E_BOUNDS, true);
    __syncthreads();
    return false;
  }
  if (c.tid == 0) c.sflag[2] = c.t;
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------- GEMV row streamer

// Streams the rows of one instruction through a per-wavefront register ring.
// Row k of this wavefront's stream is m.row(k) (K bf16 values), dotted with
// xs[m.xoff(k) .. + K); the result goes to the LDS slot m.slot(k).  The
// stream is S units of 1 KiB (one 16-byte load per lane).  Inside a ring pass
// whose refills are all needed, every refill is issued without a branch and
// nothing else touches global memory, so the compiler waits for exactly the
// oldest load instead of draining the ring; the last pass refills nothing.
// A CU's vector loads complete in issue order, so every load issued ahead of
// the next instruction's input fetch delays that fetch: the streamer issues
// no load it does not need, and the ring is only as deep as the bandwidth
// needs (8 KiB per wavefront, 64 KiB per CU in flight).
template <class Map>
struct RowStream {
  const Map& m;
  const int K, nseg, S;
  const uint32_t lane16;   // this lane's byte offset inside a 1 KiB segment
  const int lane;
  const int first;         // units 0 .. first-1 are staged in LDS, not streamed here
  int ps, pseg, pk;        // producer cursor (wave-uniform)
  const char* row;         // the producer's current row
  u32x4 ring[RING];

  __device__ __forceinline__ RowStream(const Map& m_, int K_, int nrows, int lane_, int first_ = 0)
      : m(m_), K(uni(K_)), nseg(uni((K_ + 511) >> 9)), S(uni(nrows * ((K_ + 511) >> 9))),
        lane16((uint32_t)lane_ * 16u), lane(lane_), first(uni(first_)), ps(first), pseg(first % nseg),
        pk(first / nseg) {
    row = ps < S ? (const char*)m.row(pk) : nullptr;
  }
  // Weights are read with buffer loads whose descriptor spans exactly the
  // current row (2K bytes): lanes past a ragged row's end, and refills past
  // the end of the stream in the last refilling pass (descriptor of 0 bytes),
  // read zeros without a memory access.
  __device__ __forceinline__ u32x4 next() {
    const bool live = ps < S;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), (short)0, live ? 2 * K : 0, (int)kBufFlags);
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)lane16, pseg * 1024, kNT);
    ++ps;
    if (++pseg == nseg) {
      pseg = 0;
      ++pk;
      if (ps < S) row = (const char*)m.row(pk);
    }
    return v;
  }
  // back to the first streamed unit, with the rows the map gives now (the
  // map's matrices were changed); the ring's old loads are not used
  __device__ __forceinline__ void restart() {
    ps = first;
    pseg = first % nseg;
    pk = first / nseg;
    row = ps < S ? (const char*)m.row(pk) : nullptr;
  }
  // the first min(S - first, RING) streamed units, issued before the
  // instruction's inputs are waited for
  __device__ __forceinline__ void prefetch() {
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      if (d < S - first) ring[d] = next();
      else ring[d] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  // xs must hold finite values (zero) from each row's K up to the next
  // multiple of 512: lanes past a ragged row's end multiply zero weights.
  // pre holds units 0 .. first-1 (64 lanes x 16 bytes each), already waited for.
  __device__ __forceinline__ void run(const float* xs, float* out, const u32x4* pre = nullptr) {
    const float* xl = xs + lane * 8;
    int ck = 0, cseg = 0;
    float acc0 = 0.f, acc1 = 0.f;
    auto eat = [&](const u32x4 w) {
      const float* xp = xl + m.xoff(ck) + cseg * 512;
      const f32x4 a = *(const f32x4*)xp;
      const f32x4 b = *(const f32x4*)(xp + 4);
      acc0 = fmaf(bf_lo(w.x), a.x, acc0);
      acc1 = fmaf(bf_hi(w.x), a.y, acc1);
      acc0 = fmaf(bf_lo(w.y), a.z, acc0);
      acc1 = fmaf(bf_hi(w.y), a.w, acc1);
      acc0 = fmaf(bf_lo(w.z), b.x, acc0);
      acc1 = fmaf(bf_hi(w.z), b.y, acc1);
      acc0 = fmaf(bf_lo(w.w), b.z, acc0);
      acc1 = fmaf(bf_hi(w.w), b.w, acc1);
      if (++cseg == nseg) {
        out[m.slot(ck)] = wave_sum(acc0 + acc1);
        acc0 = 0.f;
        acc1 = 0.f;
        cseg = 0;
        ++ck;
      }
    };
    for (int u = 0; u < first; ++u) eat(pre[u * 64 + lane]);
    const int R = S - first;
    for (int s0 = 0; s0 < R; s0 += RING) {
      if (s0 + RING < R) {
#pragma unroll
        for (int d = 0; d < RING; ++d) {
          eat(ring[d]);
          ring[d] = next();
        }
      } else {
#pragma unroll
        for (int d = 0; d < RING; ++d)
          if (s0 + d < R) eat(ring[d]);
      }
    }
  }
};

// zero xs[n .. n rounded up to 512) (the padding a ragged row length reads)
__device__ __forceinline__ void pad_zero(Ctx& c, float* x, int n) {
  const int end = (n + 511) & ~511;
  for (int i = n + c.tid; i < end; i += kThreads) x[i] = 0.f;
}

// rows of a tile handled by wavefront w: local rows w, w + kWaves, ...
__device__ __forceinline__ int wave_rows(int nrows, int w) {
  return nrows > w ? (nrows - w + kWaves - 1) / kWaves : 0;
}



// Rows of one GEMV instruction, described by data so that every dense
// opcode runs the same code (one copy of the streaming loop keeps the hot
// code inside the instruction cache).  Output row r in [a, a + nrows) has R
// streamed rows (R = 2 pairs gate/up or two experts); streamed row s of r
// comes from matrix part s, whose rows may be split over up to three
// pointers at global rows s1 and s2 (Wq|Wk|Wv, or expert a|expert b).
struct GemvDesc {
  const uint16_t *b00, *b01, *b02;
  const uint16_t *b10, *b11, *b12;
  int s1, s2, K, R, xoff1, a, w;
};

struct GenMap {
  const GemvDesc& g;
  __device__ __forceinline__ const uint16_t* row(int k) const {
    const bool two = g.R == 2;
    const int j = two ? (k >> 1) : k;
    const bool s = two && (k & 1);
    const int r = g.a + g.w + j * kWaves;
    const bool in1 = r >= g.s1, in2 = r >= g.s2;
    const int r0 = in2 ? g.s2 : (in1 ? g.s1 : 0);
    const uint16_t* p0 = psel(in2, psel(in1, g.b00, g.b01), g.b02);
    const uint16_t* p1 = psel(in2, psel(in1, g.b10, g.b11), g.b12);
    return psel(s, p0, p1) + (size_t)(r - r0) * g.K;
  }
  __device__ __forceinline__ int xoff(int k) const { return (g.R == 2 && (k & 1)) ? g.xoff1 : 0; }
  __device__ __forceinline__ int slot(int k) const {
    return g.R == 2 ? 2 * (g.w + (k >> 1) * kWaves) + (k & 1) : g.w + k * kWaves;
  }
};

constexpr int kNoSplit = 0x7fffffff;

// the embedding rows [r0, r1) of every sequence's token of this step, into
// dst interleaved (row r of sequence b at dst[m((r - r0) * B + b)])
template <class M = InPlace>
__device__ __forceinline__ bool embed_rows(Ctx& c, int r0, int r1, float* dst, M m = M()) {
  CKParams& p = c.p;
  if (!step_tokens(c)) return false;
  const int B = c.B;
  for (int b = 0; b < B; ++b) {
    const uint16_t* e = wptr(p, W_EMBED) + (size_t)step_tok(c)[b] * p.d;
    for (int i = r0 + c.tid; i < r1; i += kThreads) dst[m((i - r0) * B + b)] = bf_val(ld_u16(e + i));
  }
  return true;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// LM-head epilogue: logits out, and this tile's (max, lowest argmax), for
// every sequence (row i of sequence sq is out[i * NB + sq])
template <int NB>
__device__ __forceinline__ void lmhead_epilogue(Ctx& c, int a, int b, int index) {
  CKParams& p = c.p;
  for (int sq = 0; sq < NB; ++sq) {
    float* logits = p.logits_out ? p.logits_out + ((size_t)sq * p.n_steps + c.t) * p.V + a : nullptr;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int fin = 1;
    for (int i = c.tid; i < b - a; i += kThreads) {
      const float v = c.out[i * NB + sq];
      if (logits) st_f32(logits + i, v);
      fin &= isfinite(v) ? 1 : 0;
      if (better(v, a + i, bv, bi)) { bv = v; bi = a + i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      fin &= __shfl_xor(fin, off);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    int* ired = (int*)(c.red + 64);
    if (c.lane == 0) {
      c.red[c.wave] = bv;
      ired[c.wave] = bi;
      ired[16 + c.wave] = fin;
    }
    __syncthreads();
    if (c.tid == 0) {
      bv = c.red[0];
      bi = ired[0];
      bool all_fin = ired[16] != 0;
      for (int w = 1; w < kWaves; ++w) {
        if (better(c.red[w], ired[w], bv, bi)) { bv = c.red[w]; bi = ired[w]; }
        all_fin = all_fin && ired[16 + w] != 0;
      }
      if (!all_fin) raise_error(c, MKD_E_NONFINITE, false);
      const uint32_t tag = tag_of(p, c.t, p.L);
      ll_store(p.lm + (size_t)(2 * index) * NB + sq, bv, tag);
      ll_store(p.lm + (size_t)(2 * index + 1) * NB + sq, __int_as_float(bi), tag);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void desc_init(GemvDesc& g, int a, int w) {
  g.b00 = g.b01 = g.b02 = g.b10 = g.b11 = g.b12 = nullptr;
  g.s1 = g.s2 = kNoSplit;
  g.R = 1;
  g.xoff1 = 0;
  g.a = a;
  g.w = w;
}

// dense gate/up rows of layer l: output row r streams gate row r, then up row r
__device__ __forceinline__ void desc_upgate(CKParams& p, int l, GemvDesc& g) {
  g.b00 = lptr(p, l, WL_GATE);
  g.b10 = lptr(p, l, WL_UP);
  g.R = 2;
  g.K = p.d;
}

// LDS staging area of this wavefront's weight units, after the reduction scratch
__device__ __forceinline__ u32x4* pre_area(Ctx& c) {
  return (u32x4*)(c.red + kRed) + (size_t)c.wave * c.p.pre_units * 64;
}

// Stage the first stream rows of this wavefront for the dense gate/up tile
// [a, b) of layer l in LDS, as many whole rows as pre_units units (1 KiB,
// one 16-byte load per lane) hold: 16-byte loads that write LDS
// directly (lane i's bytes land at 16 i of the unit's 1 KiB), issued while the
// workgroup has nothing else in its load queue (the next instruction's weights
// loaded ahead of it, epic-kernel README, "L2 prefetching overlapped with
// prior instructions").  Rows are read through descriptors that span exactly
// the row, as in the streamer.  The wavefront waits for its staging loads
// here: it is about to wait microseconds for its next inputs anyway, and while
// such loads are outstanding the compiler makes every later LDS access wait
// for all vector memory operations.  (Staging the down projection's rows at
// the end of gate/up, and the LM head's at the end of the last down
// projection, was measured slower: every workgroup then loads at once and
// starts waiting for its inputs only after those loads.)
__device__ __forceinline__ void stage_upgate(Ctx& c, int l, int a, int b) {
  CKParams& p = c.p;
  GemvDesc g;
  desc_init(g, a, c.wave);
  desc_upgate(p, l, g);
  const GenMap m{g};
  const int nseg = (g.K + 511) >> 9;
  const int n = min(g.R * wave_rows(b - a, c.wave), p.pre_units / nseg) * nseg;   // whole rows
  __attribute__((address_space(3))) char* dst = (__attribute__((address_space(3))) char*)pre_area(c);
  int k = 0, seg = 0;
  for (int u = 0; u < n; ++u) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(m.row(k), (uint32_t)g.K * 2u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + u * 1024, 16, c.lane * 16, seg * 1024, 0, kNT);
    if (++seg == nseg) {
      seg = 0;
      ++k;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Matrices, inputs and norm gains of one dense GEMV instruction (the opcode
// picks them; everything else is shared): the row map g, the tagged inputs
// f (vector, residual rows; every sequence's, interleaved), the RMSNorm
// gains of the vector (or null) and whether the vector (layer 0 QKV) or the
// residual rows (layer 0 O-proj) come from the embedding instead.
__device__ __forceinline__ void gemv_setup(Ctx& c, int op, int l, int a, int b, uint32_t tag, GemvDesc& g,
                                           Fetch (&f)[2], const uint16_t*& gamma, bool& embed_x,
                                           bool& embed_res) {
  CKParams& p = c.p;
  desc_init(g, a, c.wave);
  gamma = nullptr;
  f[0] = {p.h, 0, tag, c.xs};
  f[1] = {p.h, 0, tag, c.res};
  embed_x = embed_res = false;
  const int B = c.B;
  switch (op) {
    case OP_QKV:
      g.b00 = lptr(p, l, WL_Q); g.b01 = lptr(p, l, WL_K); g.b02 = lptr(p, l, WL_V);
      g.s1 = p.qd; g.s2 = p.qd + p.kvd; g.K = p.d;
      gamma = lptr(p, l, WL_ATTN_NORM);
      if (l == 0) embed_x = true;
      else f[0] = {p.h, p.d * B, tag, c.xs};
      break;
    case OP_OPROJ:
      g.b00 = lptr(p, l, WL_O); g.K = p.qd;
      f[0] = {p.aout, p.qd * B, tag, c.xs};
      if (l == 0) embed_res = true;
      else f[1] = {p.h + (size_t)a * B, (b - a) * B, tag, c.res};   // published by the previous layer
      break;
    case OP_UPGATE:
      desc_upgate(p, l, g);
      gamma = lptr(p, l, WL_FFN_NORM);
      f[0] = {p.hmid, p.d * B, tag, c.xs};
      break;
    case OP_DOWN:
      g.b00 = lptr(p, l, WL_DOWN); g.K = p.F;
      f[0] = {p.act, p.F * B, tag, c.xs};
      f[1] = {p.hmid + (size_t)a * B, (b - a) * B, tag, c.res};
      break;
    default:  // OP_LMHEAD
      g.b00 = wptr(p, p.tied ? W_EMBED : W_LM_HEAD); g.K = p.d;
      gamma = wptr(p, W_FINAL_NORM);
      f[0] = {p.h, p.d * B, tag, c.xs};
      break;
  }
}

// stage the instruction's input vectors in LDS (xs, word i at xs[m(i)], and
// the residual rows in res), every sequence's interleaved; xs is zero from K
// up to the next multiple of 512 (the streamers read whole 512-element segments)
template <class M = InPlace>
__device__ __forceinline__ bool gemv_inputs(Ctx& c, int a, int b, int K, const Fetch (&f)[2], bool embed_x,
                                            bool embed_res, M m = M()) {
  CKParams& p = c.p;
  if (embed_x) {
    // the token comes from the previous step's LM-head partials (it waits on
    // them itself); the embedding row is a plain read
    if (!embed_rows(c, 0, p.d, c.xs, m)) return false;
    mark_ready(c);
    __syncthreads();
  } else {
    if (embed_res && !embed_rows(c, a, b, c.res)) return false;
    if (!gather_inputs<2, M>(c, f, m)) return false;
  }
  if (K & 511) {
    const int B = c.B;
    for (int i = K * B + c.tid; i < ((K + 511) & ~511) * B; i += kThreads) c.xs[m(i)] = 0.f;
    __syncthreads();
  }
  return true;
}

// write the instruction's outputs from the row results in LDS (row i of
// sequence sq at out[i * NB + sq]; the gate/up opcode's row i has its gate
// result at row 2i and its up result at row 2i + 1)
template <int NB>
__device__ __forceinline__ void gemv_epilogue(Ctx& c, int op, int l, int a, int b, int index, uint32_t tag) {
  CKParams& p = c.p;
  const int n = (b - a) * NB;
  const size_t o = (size_t)a * NB;
  switch (op) {
    case OP_QKV:
      for (int j = c.tid; j < n; j += kThreads) {
        const int i = j / NB, sq = j - i * NB;
        ll_store(p.qkv + (size_t)sq * p.s_qkv + a + i, c.out[j], tag);
      }
      break;
    case OP_OPROJ:
      for (int j = c.tid; j < n; j += kThreads) ll_store(p.hmid + o + j, c.res[j] + c.out[j], tag);
      break;
    case OP_UPGATE:
      for (int j = c.tid; j < n; j += kThreads) {
        const int i = j / NB, sq = j - i * NB;
        ll_store(p.act + o + j, silu(c.out[2 * i * NB + sq]) * c.out[(2 * i + 1) * NB + sq], tag);
      }
      break;
    case OP_DOWN: {
      const uint32_t otag = tag_of(p, c.t, l + 1);
      for (int j = c.tid; j < n; j += kThreads) ll_store(p.h + o + j, c.res[j] + c.out[j], otag);
      break;
    }
    default:
      lmhead_epilogue<NB>(c, a, b, index);
      break;
  }
}

// stream rows of this wavefront whose weights the previous instruction of
// the workgroup staged in LDS (gate/up only; see stage_upgate)
__device__ __forceinline__ int staged_rows(Ctx& c, int op, int ns, int nseg) {
  return op == OP_UPGATE && c.instr > 0 ? min(ns, c.p.pre_units / nseg) : 0;
}

// ---------------------------------------------------------------- expert prediction

// Speculative expert prediction (epic-kernel README, "Speculative expert
// prediction": the top-2 experts are predicted from the pre-attention
// residual before the router runs, and the predicted experts' weights are
// loaded early).  sflag words of the prediction a workgroup holds, and the
// tag of the (step, layer) it belongs to.
constexpr int kPredA = 5, kPredB = 6, kPredStamp = 7;
// route words 4 and 5: the published prediction (experts a and b as int bits)
constexpr int kPredWord = 4;

// The O-projection fetches the layer's published prediction for the gate/up
// tile that follows it: one 16-byte load of both words, requested once the
// O-projection's inputs are in (the prediction was published during the
// attention phase) and read after its outputs are stored.  A prediction
// whose words are not current, or that names no valid pair, is dropped.
__device__ __forceinline__ u32x4 pred_request(CKParams& p) {
  return __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(p.route + kPredWord, 16u), 0, 0, kSC1);
}
__device__ __forceinline__ void pred_keep(Ctx& c, const u32x4& v, uint32_t tag) {
  const int pa = (int)v.x, pb = (int)v.z;
  if (v.y == tag && v.w == tag && pa >= 0 && pa < c.p.E && pb >= 0 && pb < c.p.E && pa != pb) {
    c.sflag[kPredA] = pa;
    c.sflag[kPredB] = pb;
    c.sflag[kPredStamp] = (int)tag;
  }
}

// Any row length: rows stream through the runtime-length RowStream, the
// input vector is read from LDS per 1 KiB unit.
__device__ __forceinline__ bool op_gemv(Ctx& c, int op, int l, int a, int b, int index, bool pred_fetch = false) {
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, op == OP_LMHEAD ? p.L : l);
  GemvDesc g;
  Fetch f[2];
  const uint16_t* gamma;
  bool embed_x, embed_res;
  gemv_setup(c, op, l, a, b, tag, g, f, gamma, embed_x, embed_res);
  const GenMap m{g};
  const int nseg = (g.K + 511) >> 9;
  const int ns = g.R * wave_rows(b - a, c.wave);
  RowStream<GenMap> rs(m, g.K, ns, c.lane, staged_rows(c, op, ns, nseg) * nseg);
  rs.prefetch();
  const Gains gr = load_gains(c, p.d, gamma ? gamma : wptr(p, W_FINAL_NORM));
  if (!gemv_inputs(c, a, b, g.K, f, embed_x, embed_res)) return false;
  u32x4 pv = u32x4{0u, 0u, 0u, 0u};
  if (pred_fetch && c.tid == 0) pv = pred_request(p);
  if (gamma) rmsnorm_g(c, p.d, gamma, gr);
  // staged units were written by this wavefront, which waited for them
  rs.run(c.xs, c.out, pre_area(c));
  __syncthreads();
  gemv_epilogue<1>(c, op, l, a, b, index, tag);
  if (pred_fetch && c.tid == 0) pred_keep(c, pv, tag);
  return true;
}

// Absolute output row r of part `part` (0, or 1 for the up rows).
__device__ __forceinline__ const uint16_t* row_of(const GemvDesc& g, int r, int part) {
  const bool in1 = r >= g.s1, in2 = r >= g.s2;
  const int r0 = in2 ? g.s2 : (in1 ? g.s1 : 0);
  const uint16_t* p0 = psel(in2, psel(in1, g.b00, g.b01), g.b02);
  const uint16_t* p1 = psel(in2, psel(in1, g.b10, g.b11), g.b12);
  return psel(part != 0, p0, p1) + (size_t)(r - r0) * g.K;
}

// A wavefront's stream rows in order (output rows r0, r0 + kWaves, ...; with
// R == 2 each output row streams its gate row, then its up row), stepped by
// pointer increments except where the Q|K|V split points are crossed.
struct RowCursor {
  const GemvDesc& g;
  int r, part;
  const uint16_t* p0;
  const uint16_t* p1;
  __device__ __forceinline__ RowCursor(const GemvDesc& g_, int r0) : g(g_), r(r0), part(0) {
    p0 = row_of(g, r, 0);
    p1 = g.R == 2 ? row_of(g, r, 1) : p0;
  }
  __device__ __forceinline__ const uint16_t* next() {
    const uint16_t* q = part ? p1 : p0;
    if (g.R == 2 && part == 0) {
      part = 1;
      return q;
    }
    part = 0;
    const int nr = r + kWaves;
    const bool cross = (r < g.s1 && nr >= g.s1) || (r < g.s2 && nr >= g.s2);
    r = nr;
    if (cross) {
      p0 = row_of(g, r, 0);
      p1 = g.R == 2 ? row_of(g, r, 1) : p0;
    } else {
      p0 += (size_t)kWaves * g.K;
      p1 += (size_t)kWaves * g.K;
    }
    return q;
  }
};

// Row length NSEG x 512 (rows shorter by less than 512 read zeros past
// their end).  Each lane keeps its 8-element slices of the input vector for
// all NSEG segments in registers, so a 1 KiB weight unit costs 16 VALU
// operations and no LDS traffic, and RMSNorm runs inside each wavefront on
// those registers (every wavefront holds the whole vector) without a
// workgroup barrier.  The register ring holds RROWS rows (16 units): the
// first half is requested before the inputs are waited for, the second
// half as soon as they have arrived, so HBM keeps streaming while the
// wavefront normalises and works through the rows already on chip.  Every
// load after the inputs have arrived is issued without a branch (rows past
// the end use a zero-size descriptor), which keeps the compiler's waits
// exact: each row waits only for its own loads.
template <int NSEG>
__device__ __forceinline__ bool op_gemv_fast(Ctx& c, int op, int l, int a, int b, int index,
                                             bool pred_fetch = false) {
  constexpr int RROWS = 16 / NSEG > 1 ? 16 / NSEG : 1;
  constexpr int HROWS = RROWS / 2 > 1 ? RROWS / 2 : 1;
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, op == OP_LMHEAD ? p.L : l);
  GemvDesc g;
  Fetch f[2];
  const uint16_t* gamma;
  bool embed_x, embed_res;
  gemv_setup(c, op, l, a, b, tag, g, f, gamma, embed_x, embed_res);
  const int lane = c.lane;
  const uint32_t rbytes = (uint32_t)g.K * 2u;
  const int ns = g.R * wave_rows(b - a, c.wave);   // stream rows of this wavefront
  const int npre = staged_rows(c, op, ns, NSEG);    // ... of which staged in LDS
  const int nq = ns - npre;                         // ... and streamed through the ring
  RowCursor cur(g, a + c.wave);
  for (int i = 0; i < npre; ++i) cur.next();

  u32x4 ring[RROWS][NSEG];
  auto load_row = [&](u32x4 (&dst)[NSEG], const uint16_t* row, bool live) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, live ? rbytes : 0u);
#pragma unroll
    for (int s = 0; s < NSEG; ++s)
      dst[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, s * 1024, kNT);
  };
#pragma unroll
  for (int h = 0; h < HROWS; ++h)
    if (h < nq) load_row(ring[h], cur.next(), true);
  // norm gains for this lane's slices (zeros past d)
  u32x4 gv[NSEG];
  if (gamma) {
    const __amdgpu_buffer_rsrc_t gr = make_rsrc(gamma, (uint32_t)p.d * 2u);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) gv[s] = __builtin_amdgcn_raw_buffer_load_b128(gr, (s * 512 + lane * 8) * 2, 0, 0);
  }
  if (!gemv_inputs(c, a, b, g.K, f, embed_x, embed_res)) return false;
  // everything requested so far has arrived (it was issued before the
  // inputs, and loads complete in order); saying so keeps the waits below exact
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  u32x4 pv = u32x4{0u, 0u, 0u, 0u};
  if (pred_fetch && c.tid == 0) pv = pred_request(p);
  const bool deep = nq > HROWS;
  if (deep) {
#pragma unroll
    for (int h = HROWS; h < RROWS; ++h) load_row(ring[h], cur.next(), h < nq);
  }

  float x[NSEG][8];
#pragma unroll
  for (int s = 0; s < NSEG; ++s) {
    const f32x4 u = *(const f32x4*)(c.xs + s * 512 + lane * 8);
    const f32x4 v = *(const f32x4*)(c.xs + s * 512 + lane * 8 + 4);
    x[s][0] = u.x; x[s][1] = u.y; x[s][2] = u.z; x[s][3] = u.w;
    x[s][4] = v.x; x[s][5] = v.y; x[s][6] = v.z; x[s][7] = v.w;
  }
  if (gamma) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NSEG; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(x[s][i], x[s][i], ss);
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)p.d + p.eps);
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const uint32_t gw[4] = {gv[s].x, gv[s].y, gv[s].z, gv[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[s][2 * i] = (x[s][2 * i] * inv) * bf_lo(gw[i]);
        x[s][2 * i + 1] = (x[s][2 * i + 1] * inv) * bf_hi(gw[i]);
      }
    }
  }
  auto dot_row = [&](const u32x4 (&w)[NSEG]) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      a0 = fmaf(bf_lo(w[s].x), x[s][0], a0);
      a1 = fmaf(bf_hi(w[s].x), x[s][1], a1);
      a0 = fmaf(bf_lo(w[s].y), x[s][2], a0);
      a1 = fmaf(bf_hi(w[s].y), x[s][3], a1);
      a0 = fmaf(bf_lo(w[s].z), x[s][4], a0);
      a1 = fmaf(bf_hi(w[s].z), x[s][5], a1);
      a0 = fmaf(bf_lo(w[s].w), x[s][6], a0);
      a1 = fmaf(bf_hi(w[s].w), x[s][7], a1);
    }
    return wave_sum(a0 + a1);
  };
  // LDS slot of stream row k; every lane writes the same value to it
  const GenMap m{g};
  // rows staged in LDS (written by this wavefront, which waited for them)
  const u32x4* pre = pre_area(c);
  for (int q = 0; q < npre; ++q) {
    u32x4 w[NSEG];
#pragma unroll
    for (int s = 0; s < NSEG; ++s) w[s] = pre[(q * NSEG + s) * 64 + lane];
    c.out[m.slot(q)] = dot_row(w);
  }
  if (!deep) {
#pragma unroll
    for (int h = 0; h < HROWS; ++h)
      if (h < nq) c.out[m.slot(npre + h)] = dot_row(ring[h]);
  } else {
    int q0 = 0;
    for (; q0 + 2 * RROWS <= nq; q0 += RROWS) {   // every refill is a live row
#pragma unroll
      for (int h = 0; h < RROWS; ++h) {
        c.out[m.slot(npre + q0 + h)] = dot_row(ring[h]);
        load_row(ring[h], cur.next(), true);
      }
    }
    if (q0 + RROWS < nq) {                          // last refilling pass
#pragma unroll
      for (int h = 0; h < RROWS; ++h) {
        c.out[m.slot(npre + q0 + h)] = dot_row(ring[h]);
        load_row(ring[h], cur.next(), q0 + RROWS + h < nq);
      }
      q0 += RROWS;
    }
#pragma unroll
    for (int h = 0; h < RROWS; ++h)                 // drain
      if (q0 + h < nq) c.out[m.slot(npre + q0 + h)] = dot_row(ring[h]);
  }
  __syncthreads();
  gemv_epilogue<1>(c, op, l, a, b, index, tag);
  if (pred_fetch && c.tid == 0) pred_keep(c, pv, tag);
  return true;
}

// ---------------------------------------------------------------- several sequences

// RMSNorm gains of the batched path: this thread's 8-element slices s = tid
// and s = tid + kThreads (d <= 16 kThreads), 16 bytes each, read before the
// inputs are waited for.
struct SliceGains {
  u32x4 g[2];
};
__device__ __forceinline__ SliceGains load_slice_gains(Ctx& c, int d, const uint16_t* gamma) {
  SliceGains r;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(gamma, (uint32_t)d * 2u);
#pragma unroll
  for (int k = 0; k < 2; ++k) r.g[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c.tid + k * kThreads) * 16, 0, 0);
  return r;
}

// Sequence b's vector (element k at xs[SlicePad(k NB + b)]) <- its RMSNorm
// times gamma.  Each thread takes whole 8-element slices (8 NB floats, read
// and written as 16-byte vectors; consecutive threads' slices are an odd
// number of 16-byte units apart, so the accesses spread over all LDS banks).
// An element-by-element pass over this layout hit a handful of banks and
// cost 6 us per instruction at NB = 8.  Needs d % 8 == 0 and d <= 16 kThreads.
template <int NB>
__device__ __forceinline__ void rmsnorm_b(Ctx& c, int d, const SliceGains& sg) {
  constexpr int XS = SlicePad<NB>::kStride, V = 2 * NB;   // f32x4 vectors per slice
  const int nsl = d >> 3;
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ss[b] = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int sl = c.tid + k * kThreads;
    if (sl < nsl) {
      const f32x4* v = (const f32x4*)(c.xs + sl * XS);
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const f32x4 u = v[q];
        ss[(4 * q + 0) % NB] = fmaf(u.x, u.x, ss[(4 * q + 0) % NB]);
        ss[(4 * q + 1) % NB] = fmaf(u.y, u.y, ss[(4 * q + 1) % NB]);
        ss[(4 * q + 2) % NB] = fmaf(u.z, u.z, ss[(4 * q + 2) % NB]);
        ss[(4 * q + 3) % NB] = fmaf(u.w, u.w, ss[(4 * q + 3) % NB]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float w = wave_sum(ss[b]);
    if (c.lane == 0) c.red[b * kWaves + c.wave] = w;
  }
  __syncthreads();
  float inv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += c.red[b * kWaves + w];
    inv[b] = 1.0f / sqrtf(tot / (float)d + c.p.eps);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int sl = c.tid + k * kThreads;
    if (sl < nsl) {
      f32x4* v = (f32x4*)(c.xs + sl * XS);
      const uint32_t gw[4] = {sg.g[k].x, sg.g[k].y, sg.g[k].z, sg.g[k].w};
      float g[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[2 * e] = bf_lo(gw[e]);
        g[2 * e + 1] = bf_hi(gw[e]);
      }
#pragma unroll
      for (int q = 0; q < V; ++q) {
        f32x4 u = v[q];
        u.x = (u.x * inv[(4 * q + 0) % NB]) * g[(4 * q + 0) / NB];
        u.y = (u.y * inv[(4 * q + 1) % NB]) * g[(4 * q + 1) / NB];
        u.z = (u.z * inv[(4 * q + 2) % NB]) * g[(4 * q + 2) / NB];
        u.w = (u.w * inv[(4 * q + 3) % NB]) * g[(4 * q + 3) / NB];
        v[q] = u;
      }
    }
  }
  __syncthreads();
}

// Rows of one instruction dotted with NB input vectors at once.  The inputs
// sit interleaved in LDS (element k of sequence b at xs[SlicePad(k NB + b)]),
// so the slice a lane needs for one 16-byte weight load (8 elements) is 8 NB
// contiguous floats, and consecutive lanes' slices start on different banks.  The workgroup's 8 wavefronts form a WR x WS grid over
// the tile: wavefront (wr, ws) takes stream rows wr, wr + WR, ... and
// segments ws, ws + WS, ...  A tile with many rows keeps whole rows per
// wavefront (WS = 1); a tile with few rows (QKV, O-proj and down tiles are
// 8-12 rows) also splits K, so that every wavefront still has rows to group
// and loads to keep in flight, and the WS partial sums of a row are added in
// LDS afterwards, in a fixed order.  A wavefront walks its rows in groups of
// G, segment by segment: one ring step holds the G rows' units of one
// segment, and one read of the input slice serves all G (LDS traffic per
// weight byte falls G-fold).  The ring is D steps deep (12 KiB per
// wavefront); DPRE steps are requested before the inputs are waited for
// (all of them measured best: deeper rings and later refills were slower).
// Loads past the wavefront's last row use zero-size descriptors, so every
// refill is issued without a branch.
// How a batched GEMV instruction's ns rows of nseg 512-element segments are
// split over the wavefronts: a WR x WS grid, wavefront (wr, ws) takes rows
// wr, wr + WR, ... and segments ws, ws + WS, ... of [s0, s1); it streams
// them in steps of kBatchRows rows by one segment, row groups outermost.
constexpr int kBatchRows = 4;
struct BatchGrid {
  int WR, WS, wr, ws, nrow, nsw, steps;
  __device__ __forceinline__ BatchGrid(int ns, int nseg, int wave, int s0, int s1) {
    WR = kWaves;
    WS = 1;
    while (WR > 1 && ns < 4 * WR && 2 * WS <= nseg) {
      WR >>= 1;
      WS <<= 1;
    }
    wr = wave / WS;
    ws = wave % WS;
    nrow = ns > wr ? (ns - wr + WR - 1) / WR : 0;
    const int span = s1 - s0;
    nsw = span > ws ? (span - ws + WS - 1) / WS : 0;
    steps = ((nrow + kBatchRows - 1) / kBatchRows) * nsw;
  }
};

// This wavefront's gate/up units staged in LDS (several sequences): they sit
// in the input area, past the inputs of gate/up and of the O-projection
__device__ __forceinline__ u32x4* pre_area_b(Ctx& c) {
  return (u32x4*)(c.xs + c.p.pre_off) + (size_t)c.wave * c.p.pre_units * 64;
}

template <int NB>
struct BatchStream {
  static constexpr int G = kBatchRows, D = 3, DPRE = 3;
  const GemvDesc& g;
  const int K, nseg, ns;
  int WR, WS, wr, ws, nrow, nsw, steps;
  const int U;                      // leading steps already staged in LDS (gate/up)
  const uint32_t lane16;
  int pg, pi;                       // producer: row group, segment (of this wavefront's)
  __amdgpu_buffer_rsrc_t pr[G];     // the producer group's row descriptors
  u32x4 ring[D][G];

  // Segments [s0, s1) of every row (one pass; the input slice of segment s
  // is at xs + (s - s0) * 512 NB).  The wavefront grid depends on the whole
  // row length, so every pass of an instruction splits the work alike.  The
  // first U steps of this wavefront were loaded into LDS beforehand, in
  // step order (stage_upgate_b); the stream starts after them.
  const int s0;
  __device__ __forceinline__ BatchStream(const GemvDesc& g_, int ns_, int wave, int lane, int s0_, int s1_,
                                         int staged = 0)
      : g(g_), K(uni(g_.K)), nseg(uni((g_.K + 511) >> 9)), ns(uni(ns_)), U(uni(staged)),
        lane16((uint32_t)lane * 16u), pg(0), pi(0), s0(uni(s0_)) {
    const BatchGrid q(ns, nseg, wave, s0, uni(s1_));
    WR = q.WR; WS = q.WS; wr = q.wr; ws = q.ws; nrow = q.nrow; nsw = q.nsw; steps = q.steps;
    if (U > 0) {
      pg = U / nsw;
      pi = U - pg * nsw;
    }
    set_group();
  }
  // stream row k of the tile: output row a + k (or a + k/2, gate or up)
  __device__ __forceinline__ const uint16_t* row(int k) const {
    return g.R == 2 ? row_of(g, g.a + (k >> 1), k & 1) : row_of(g, g.a + k, 0);
  }
  __device__ __forceinline__ void set_group() {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const int i = pg * G + r;
      const bool live = i < nrow;
      pr[r] = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row(live ? wr + i * WR : 0)), (short)0,
                                                live ? 2 * K : 0, (int)kBufFlags);
    }
  }
  __device__ __forceinline__ void issue(u32x4 (&dst)[G]) {
    const int seg = s0 + ws + pi * WS;
#pragma unroll
    for (int r = 0; r < G; ++r)
      dst[r] = __builtin_amdgcn_raw_buffer_load_b128(pr[r], (int)lane16, seg * 1024, kNT);
    if (++pi == nsw) {
      pi = 0;
      ++pg;
      set_group();
    }
  }
  __device__ __forceinline__ void prefetch() {
#pragma unroll
    for (int d = 0; d < DPRE; ++d) issue(ring[d]);
  }
  // after the inputs have arrived
  __device__ __forceinline__ void prefetch_rest() {
#pragma unroll
    for (int d = DPRE; d < D; ++d) issue(ring[d]);
  }
  // Row results: out[k * NB + b] when WS == 1, else this wavefront's partial
  // at out[(ns + ws * ns + k) * NB + b] (combine() adds them up); a pass after
  // the first adds to what the earlier passes left there.
  __device__ __forceinline__ void run(const float* xs, float* out, bool add, const u32x4* pre = nullptr) {
    constexpr int XS = SlicePad<NB>::kStride;
    const float* xl = xs + lane16 / 16u * XS;   // this lane's slice of segment s0
    float acc[G][NB];
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
    int ci = 0, cg = 0;
    float* const dst = WS == 1 ? out : out + (size_t)(ns + ws * ns) * NB;
    if (nsw == 0 && !add) {
      // a first pass with no segment for this wavefront: its rows' sums start at zero
      for (int i = 0; i < nrow; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) dst[(wr + i * WR) * NB + b] = 0.f;
    }
    auto eat = [&](const u32x4 (&w)[G]) {
      const f32x4* xp = (const f32x4*)(xl + (ws + ci * WS) * 64 * XS);
      float x[8 * NB];
#pragma unroll
      for (int q = 0; q < 2 * NB; ++q) {
        const f32x4 v = xp[q];
        x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const uint32_t wv[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float wj = (j & 1) ? bf_hi(wv[j >> 1]) : bf_lo(wv[j >> 1]);
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = fmaf(wj, x[j * NB + b], acc[r][b]);
        }
      }
      if (++ci == nsw) {
        // the G x NB sums, four at a time; the first lane of row rr holds
        // value 4q + kQuadValue[rr] of the group (row-major over (row, sequence))
        const int rr = (int)(lane16 >> 8);
        const bool writer = ((lane16 >> 4) & 15u) == 0;
#pragma unroll
        for (int q = 0; q < G * NB / 4; ++q) {
          const float v = quad_sum(acc[(4 * q) / NB][(4 * q) % NB], acc[(4 * q + 1) / NB][(4 * q + 1) % NB],
                                   acc[(4 * q + 2) / NB][(4 * q + 2) % NB], acc[(4 * q + 3) / NB][(4 * q + 3) % NB]);
          const int vi = 4 * q + (rr == 1 ? 2 : (rr == 2 ? 1 : rr));
          const int r = vi / NB, bq = vi - r * NB;
          const int i = cg * G + r;
          if (writer && i < nrow) {
            float* o = dst + (wr + i * WR) * NB + bq;
            *o = add ? *o + v : v;
          }
        }
#pragma unroll
        for (int r = 0; r < G; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
        ci = 0;
        ++cg;
      }
    };
    for (int s = 0; s < U; ++s) {
      u32x4 w[G];
#pragma unroll
      for (int r = 0; r < G; ++r) w[r] = pre[(s * G + r) * 64 + (lane16 >> 4)];
      eat(w);
    }
    const int rs = steps - U;
    for (int s0 = 0; s0 < rs; s0 += D) {
      if (s0 + D < rs) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          eat(ring[d]);
          issue(ring[d]);
        }
      } else {
#pragma unroll
        for (int d = 0; d < D; ++d)
          if (s0 + d < rs) eat(ring[d]);
      }
    }
  }
  // out[j] = sum over the WS segment groups of their partials (after a barrier)
  __device__ __forceinline__ void combine(Ctx& c, float* out) const {
    if (WS == 1) return;
    for (int j = c.tid; j < ns * NB; j += kThreads) {
      float v = 0.f;
      for (int q = 0; q < WS; ++q) v += out[(size_t)(ns + q * ns) * NB + j];
      out[j] = v;
    }
    __syncthreads();
  }
};

// One dense GEMV instruction for NB sequences: the same rows, inputs and
// epilogues as with one sequence, every activation interleaved by sequence.
template <int NB>
__device__ __forceinline__ bool op_gemv_b(Ctx& c, int op, int l, int a, int b, int index) {
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, op == OP_LMHEAD ? p.L : l);
  GemvDesc g;
  Fetch f[2];
  const uint16_t* gamma;
  bool embed_x, embed_res;
  gemv_setup(c, op, l, a, b, tag, g, f, gamma, embed_x, embed_res);
  // The input vectors of all NB sequences must sit in LDS at once.  When
  // they do not fit (the down projection's d_ff-long input at large NB), the
  // row stream runs in passes over K, each with its slice of the inputs.
  const int nseg = (g.K + 511) >> 9;
  const SlicePad<NB> xm;
  const int pseg = uni(min(nseg, p.x_floats / (64 * SlicePad<NB>::kStride)));   // segments per pass
  const int ns = g.R * (b - a);
  if (pseg < nseg && (gamma || embed_x)) {
    // RMSNorm needs the whole vector at once; the host sizes the input area
    // so that only the down projection's input is ever split
    if (c.tid == 0) raise_error(c, MKD_E_BOUNDS, true);
    return false;
  }
  const int k1 = min(g.K, pseg * 512);
  f[0].n = k1 * NB;
  // gate/up steps the previous instruction staged in LDS (stage_upgate_b)
  const int staged = op == OP_UPGATE && c.instr > 0 && pseg == nseg
                         ? min(BatchGrid(ns, nseg, c.wave, 0, nseg).steps, p.pre_units / kBatchRows)
                         : 0;
  BatchStream<NB> bs(g, ns, c.wave, c.lane, 0, pseg, staged);
  bs.prefetch();
  const SliceGains sg = load_slice_gains(c, p.d, gamma ? gamma : wptr(p, W_FINAL_NORM));
  if (!gemv_inputs(c, a, b, k1, f, embed_x, embed_res, xm)) return false;
  // everything requested so far has arrived (loads complete in order);
  // saying so keeps the waits of the row loop exact
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  bs.prefetch_rest();
  if (gamma) rmsnorm_b<NB>(c, p.d, sg);
  bs.run(c.xs, c.out, false, pre_area_b(c));
  for (int sa = pseg; sa < nseg; sa += pseg) {
    const int sb = min(nseg, sa + pseg);
    const int ka = sa * 512, kb = min(g.K, sb * 512);
    BatchStream<NB> next(g, ns, c.wave, c.lane, sa, sb);
    next.prefetch();
    __syncthreads();  // every wavefront is done with the previous slice
    ll_fetch(c, f[0].src + (size_t)ka * NB, (kb - ka) * NB, tag, c.xs, xm);
    for (int i = (kb - ka) * NB + c.tid; i < (sb - sa) * 512 * NB; i += kThreads) c.xs[xm(i)] = 0.f;
    if (!sync_ok(c)) return false;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    next.prefetch_rest();
    next.run(c.xs, c.out, true);
  }
  __syncthreads();
  bs.combine(c, c.out);
  gemv_epilogue<NB>(c, op, l, a, b, index, tag);
  return true;
}

// Several sequences: load the first steps of this wavefront's share of a
// gate/up instruction [a, b) of layer l into LDS, in the order the batched
// streamer consumes them (BatchGrid), as many whole steps of kBatchRows
// 1 KiB units as pre_units holds.  Same timing as stage_upgate.
__device__ __forceinline__ void stage_upgate_b(Ctx& c, int l, int a, int b) {
  CKParams& p = c.p;
  GemvDesc g;
  desc_init(g, a, c.wave);
  desc_upgate(p, l, g);
  const int nseg = (g.K + 511) >> 9;
  const BatchGrid q(2 * (b - a), nseg, c.wave, 0, nseg);
  const int n = min(q.steps, p.pre_units / kBatchRows);
  __attribute__((address_space(3))) char* dst = (__attribute__((address_space(3))) char*)pre_area_b(c);
  int pg = 0, pi = 0;
  for (int j = 0; j < n; ++j) {
    const int seg = q.ws + pi * q.WS;
#pragma unroll
    for (int r = 0; r < kBatchRows; ++r) {
      const int i = pg * kBatchRows + r;
      if (i < q.nrow) {
        const int k = q.wr + i * q.WR;   // row k of the tile: gate or up row a + k/2
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(row_of(g, a + (k >> 1), k & 1), (uint32_t)g.K * 2u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + (j * kBatchRows + r) * 1024, 16, c.lane * 16,
                                                 seg * 1024, 0, kNT);
      }
    }
    if (++pi == q.nsw) {
      pi = 0;
      ++pg;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// dense GEMV opcodes: several sequences (batched kernel) by their count;
// one sequence by the compile-time row length when there is one
template <bool BATCHED>
__device__ __forceinline__ bool op_gemv_any(Ctx& c, int op, int l, int a, int b, int index,
                                            bool pred_fetch = false) {
  CKParams& p = c.p;
  if constexpr (BATCHED) {
    switch (c.B) {
      case 2: return op_gemv_b<2>(c, op, l, a, b, index);
      case 3: return op_gemv_b<3>(c, op, l, a, b, index);
      case 4: return op_gemv_b<4>(c, op, l, a, b, index);
      case 5: return op_gemv_b<5>(c, op, l, a, b, index);
      case 6: return op_gemv_b<6>(c, op, l, a, b, index);
      case 7: return op_gemv_b<7>(c, op, l, a, b, index);
      default: return op_gemv_b<8>(c, op, l, a, b, index);
    }
  }
  const int K = op == OP_OPROJ ? p.qd : (op == OP_DOWN ? p.F : p.d);
  switch ((K + 511) >> 9) {
    case 1: return op_gemv_fast<1>(c, op, l, a, b, index, pred_fetch);
    case 2: return op_gemv_fast<2>(c, op, l, a, b, index, pred_fetch);
    case 4: return op_gemv_fast<4>(c, op, l, a, b, index, pred_fetch);
    case 6: return op_gemv_fast<6>(c, op, l, a, b, index, pred_fetch);
    case 8: return op_gemv_fast<8>(c, op, l, a, b, index, pred_fetch);
    default: return op_gemv(c, op, l, a, b, index, pred_fetch);
  }
}

// ---------------------------------------------------------------- opcodes: MoE

// counts of the expert prediction's outcomes, in int words of the reduction scratch
constexpr int kSpecHitWord = 252, kSpecNWord = 253;
// The route of a layer (experts a and b as int bits, their weights) in words
// kRouteWords .. + 3 of the reduction scratch, and at kRouteStamp the tag of
// the step and layer it belongs to (0: none yet)
constexpr int kRouteWords = 8, kRouteStamp = 12;

// The expert whose gate/up rows the tile [a, b) of a layer's stacked
// (expert a, expert b) rows reads, given the two experts; -1 if the tile
// straddles both
__device__ __forceinline__ int tile_expert(CKParams& p, int a, int b, int ea, int eb) {
  return b <= p.F ? ea : (a >= p.F ? eb : -1);
}

// The stream map of this wavefront's gate/up rows of MoE tile [a, b) of
// layer l for experts (ea, eb): output row r < F is expert ea's row r, else
// expert eb's row r - F; streamed rows alternate gate and up
__device__ __forceinline__ void desc_moe_upgate(CKParams& p, int l, int a, int w, int ea, int eb, GemvDesc& g) {
  g.b00 = lptr(p, l, WL_EXPERTS + ea); g.b01 = lptr(p, l, WL_EXPERTS + eb); g.b02 = nullptr;
  g.b10 = lptr(p, l, WL_EXPERTS + p.E + ea); g.b11 = lptr(p, l, WL_EXPERTS + p.E + eb); g.b12 = nullptr;
  g.s1 = p.F; g.s2 = kNoSplit; g.K = p.d; g.R = 2; g.xoff1 = 0; g.a = a; g.w = w;
}

// One workgroup per layer, the one holding O-projection tile 0 (it waits out
// the attention phase anyway), predicts the layer's two experts and publishes
// them for the gate/up tiles: the layer's input residual h (published before
// the attention phase; for layer 0 the embedding row), RMSNorm with the FFN
// norm's gains, router logits with one expert row per wavefront, and the top
// two in the router's order and tie rule, in route words 4 and 5.
__device__ __forceinline__ bool predict_publish(Ctx& c, int l) {
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, l);
  const uint16_t* gamma = lptr(p, l, WL_FFN_NORM);
  const Gains gr = load_gains(c, p.d, gamma);
  constexpr int RU = 8;
  const uint16_t* wr = lptr(p, l, WL_ROUTER);
  const bool mine = c.wave < p.E;
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(wr + (size_t)(mine ? c.wave : 0) * p.d, mine ? (uint32_t)p.d * 2u : 0u);
  u32x4 rw[RU];
#pragma unroll
  for (int k = 0; k < RU; ++k) rw[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (k * 64 + c.lane) * 16, 0, 0);
  if (l == 0) {
    if (!embed_rows(c, 0, p.d, c.xs)) return false;
    __syncthreads();
  } else {
    const Fetch f[1] = {{p.h, p.d, tag, c.xs}};
    if (!gather<1>(c, f)) return false;
  }
  rmsnorm_g(c, p.d, gamma, gr);
  if (p.d & 511) {
    pad_zero(c, c.xs, p.d);
    __syncthreads();
  }
  if (mine) {
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < RU; ++k) {
      const int i0 = (k * 64 + c.lane) * 8;
      if (i0 < p.d) {
        const uint32_t wv[4] = {rw[k].x, rw[k].y, rw[k].z, rw[k].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(bf_lo(wv[j]), c.xs[i0 + 2 * j], acc);
          acc = fmaf(bf_hi(wv[j]), c.xs[i0 + 2 * j + 1], acc);
        }
      }
    }
    const float z = wave_sum(acc);
    if (c.lane == 0) c.red[64 + c.wave] = z;
  }
  __syncthreads();
  if (c.tid == 0) {
    int ea = 0;
    for (int e = 1; e < p.E; ++e)
      if (c.red[64 + e] > c.red[64 + ea]) ea = e;
    int eb = ea == 0 ? 1 : 0;
    for (int e = 0; e < p.E; ++e)
      if (e != ea && c.red[64 + e] > c.red[64 + eb]) eb = e;
    ll_store(p.route + kPredWord, __int_as_float(ea), tag);
    ll_store(p.route + kPredWord + 1, __int_as_float(eb), tag);
  }
  __syncthreads();
  return true;
}

__device__ __forceinline__ bool op_moe_upgate(Ctx& c, int l, int a, int b, int index) {
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, l);
  const uint16_t* gamma = lptr(p, l, WL_FFN_NORM);
  const Gains gr = load_gains(c, p.d, gamma);
  // Router logits, one wavefront per expert row.  With d <= 4096 and at most
  // one expert per wavefront the row is requested with 16-byte loads before
  // the inputs are waited for (element (k * 64 + lane) * 8 + j of the row in
  // unit k, lane's j-th value); read element by element after the wait, the
  // loads were dozens of round trips through a memory system busy with
  // other workgroups' streams.
  constexpr int RU = 8;
  const uint16_t* wr = lptr(p, l, WL_ROUTER);
  const bool router_early = p.d <= RU * 512 && p.E <= kWaves;
  u32x4 rw[RU];
  {
    const bool mine = router_early && c.wave < p.E;
    const __amdgpu_buffer_rsrc_t rr =
        make_rsrc(wr + (size_t)(mine ? c.wave : 0) * p.d, mine ? (uint32_t)p.d * 2u : 0u);
#pragma unroll
    for (int k = 0; k < RU; ++k) rw[k] = __builtin_amdgcn_raw_buffer_load_b128(rr, (k * 64 + c.lane) * 16, 0, 0);
  }
  // With a prediction for this layer (fetched by the O-projection before
  // it), the predicted expert's rows of this tile are requested before the
  // inputs are waited for; the router then decides whether they are used.
  int pa = -1, pb = -1;
  if (p.predict && uni(c.sflag[kPredStamp]) == (int)tag) {
    pa = uni(c.sflag[kPredA]);
    pb = uni(c.sflag[kPredB]);
  }
  const int tp = pa >= 0 ? tile_expert(p, a, b, pa, pb) : -1;
  GemvDesc g;
  desc_moe_upgate(p, l, a, c.wave, tp >= 0 ? pa : 0, tp >= 0 ? pb : 1, g);
  const GenMap m{g};
  RowStream<GenMap> rs(m, p.d, 2 * wave_rows(b - a, c.wave), c.lane);
  if (tp >= 0) rs.prefetch();
  const Fetch f[1] = {{p.hmid, p.d, tag, c.xs}};
  if (!gather_inputs<1>(c, f)) return false;
  rmsnorm_g(c, p.d, gamma, gr);
  if (p.d & 511) {
    pad_zero(c, c.xs, p.d);
    __syncthreads();
  }
  if (router_early) {
    if (c.wave < p.E) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < RU; ++k) {
        const int i0 = (k * 64 + c.lane) * 8;
        if (i0 < p.d) {
          const uint32_t wv[4] = {rw[k].x, rw[k].y, rw[k].z, rw[k].w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc = fmaf(bf_lo(wv[j]), c.xs[i0 + 2 * j], acc);
            acc = fmaf(bf_hi(wv[j]), c.xs[i0 + 2 * j + 1], acc);
          }
        }
      }
      const float z = wave_sum(acc);
      if (c.lane == 0) c.red[64 + c.wave] = z;
    }
  } else {
    for (int e = c.wave; e < p.E; e += kWaves) {
      float acc = 0.f;
      for (int i = c.lane; i < p.d; i += 64) acc = fmaf(bf_val(ld_u16(wr + (size_t)e * p.d + i)), c.xs[i], acc);
      const float z = wave_sum(acc);
      if (c.lane == 0) c.red[64 + e] = z;
    }
  }
  __syncthreads();
  if (c.tid == 0) {
    // top-2: larger logit first, lower expert index on ties
    int ea = 0;
    for (int e = 1; e < p.E; ++e)
      if (c.red[64 + e] > c.red[64 + ea]) ea = e;
    int eb = ea == 0 ? 1 : 0;
    for (int e = 0; e < p.E; ++e)
      if (e != ea && c.red[64 + e] > c.red[64 + eb]) eb = e;
    const float za = c.red[64 + ea], zb = c.red[64 + eb];
    const float q = expf(zb - za);
    c.sflag[3] = ea;
    c.sflag[4] = eb;
    // the route stays in LDS for this workgroup's down-projection tile of
    // the layer; the first gate/up tile publishes it for the others
    float* rt = c.red + kRouteWords;
    rt[0] = __int_as_float(ea);
    rt[1] = __int_as_float(eb);
    rt[2] = 1.0f / (1.0f + q);
    rt[3] = q / (1.0f + q);
    c.red[kRouteStamp] = __uint_as_float(tag);
    if (index == 0)
      for (int k = 0; k < 4; ++k) ll_store(p.route + k, rt[k], tag);
  }
  __syncthreads();
  const int ea = uni(c.sflag[3]), eb = uni(c.sflag[4]);
  // The requested rows are used only when they are the routed expert's (the
  // router decides; the prediction only moved some loads earlier); else the
  // stream starts again on the routed expert's rows.
  const bool hit = tp >= 0 && tp == tile_expert(p, a, b, ea, eb);
  if (tp >= 0 && c.tid == 0) {
    int* cnt = (int*)c.red;
    cnt[kSpecHitWord] += hit ? 1 : 0;
    cnt[kSpecNWord] += 1;
  }
  if (!hit) {
    desc_moe_upgate(p, l, a, c.wave, ea, eb, g);
    rs.restart();
    rs.prefetch();
  }
  rs.run(c.xs, c.out);
  __syncthreads();
  for (int i = c.tid; i < b - a; i += kThreads)
    ll_store(p.act + a + i, silu(c.out[2 * i]) * c.out[2 * i + 1], tag);
  return true;
}

__device__ __forceinline__ bool op_moe_down(Ctx& c, int l, int a, int b) {
  CKParams& p = c.p;
  const uint32_t tag = tag_of(p, c.t, l);
  const int Fpad = (p.F + 511) & ~511;
  float* rt = c.red + kRouteWords;
  // When this workgroup ran a gate/up tile of the layer, the route is already
  // in LDS: the experts' rows are then requested before the activations are
  // waited for (expert widths of whole 512-element segments; Mixtral-shaped
  // decode 4590-4625 against 4635-4704 us/token).  Otherwise the route is
  // fetched with the activations.
  const bool own = (p.F & 511) == 0 && __float_as_uint(c.red[kRouteStamp]) == tag;
  if (p.F & 511) {
    const Fetch f[4] = {{p.route, 4, tag, rt}, {p.act, p.F, tag, c.xs},
                        {p.act + p.F, p.F, tag, c.xs + Fpad}, {p.hmid + a, b - a, tag, c.res}};
    pad_zero(c, c.xs, p.F);
    pad_zero(c, c.xs + Fpad, p.F);
    if (!gather_inputs<4>(c, f)) return false;
  } else if (!own) {
    // both experts' activations are one contiguous span, in the same layout
    // in LDS: one fetch, 16 loads per thread per round trip (two round trips
    // for Mixtral's 2 x 14336 words, against a dozen in 2048-word pieces)
    const Fetch f[3] = {{p.act, 2 * p.F, tag, c.xs}, {p.hmid + a, b - a, tag, c.res}, {p.route, 4, tag, rt}};
    if (!gather_inputs<3, InPlace, 16>(c, f)) return false;
  }
  const int ea = uni(__float_as_int(rt[0])), eb = uni(__float_as_int(rt[1]));
  const float wa = __int_as_float(uni(__float_as_int(rt[2])));
  const float wb = __int_as_float(uni(__float_as_int(rt[3])));
  if (ea < 0 || ea >= p.E || eb < 0 || eb >= p.E) {
    if (c.tid == 0) raise_error(c, MKD_E_BOUNDS, true);
    __syncthreads();
    return false;
  }
  GemvDesc g;
  g.b00 = lptr(p, l, WL_EXPERTS + 2 * p.E + ea); g.b01 = g.b02 = nullptr;
  g.b10 = lptr(p, l, WL_EXPERTS + 2 * p.E + eb); g.b11 = g.b12 = nullptr;
  g.s1 = g.s2 = kNoSplit; g.K = p.F; g.R = 2; g.xoff1 = Fpad; g.a = a; g.w = c.wave;
  const GenMap m{g};
  RowStream<GenMap> rs(m, p.F, 2 * wave_rows(b - a, c.wave), c.lane);
  rs.prefetch();
  if (own) {
    // (the rows requested above are in flight meanwhile)
    const Fetch f[2] = {{p.act, 2 * p.F, tag, c.xs}, {p.hmid + a, b - a, tag, c.res}};
    if (!gather_inputs<2, InPlace, 16>(c, f)) return false;
  }
  rs.run(c.xs, c.out);
  __syncthreads();
  const uint32_t otag = tag_of(p, c.t, l + 1);
  for (int i = c.tid; i < b - a; i += kThreads)
    ll_store(p.h + a + i, c.res[i] + (wa * c.out[2 * i] + wb * c.out[2 * i + 1]), otag);
  return true;
}

// ---------------------------------------------------------------- opcode: RoPE + KV append + attention

// online-softmax state of one lane group for G heads (log2 domain)
template <int G>
struct AttnState {
  float m[G], l[G], o[G][8];
};

template <int G>
__device__ __forceinline__ void merge_into(AttnState<G>& s, const float* om, const float* ol,
                                           const float (*oo)[8]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = fmaxf(s.m[g], om[g]);
    if (M == -INFINITY) continue;
    const float a1 = exp2f(s.m[g] - M), a2 = exp2f(om[g] - M);
    s.l[g] = s.l[g] * a1 + ol[g] * a2;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.o[g][i] = s.o[g][i] * a1 + oo[g][i] * a2;
    s.m[g] = M;
  }
}

// Attention of q heads q0 .. q0 + G - 1 (all of kv head kvh's, or one of
// them) over one chunk; the instruction may append K/V at pos only when it is
// the one instruction of its kv head that owns it (may_append).
template <int HD, int G>
__device__ __forceinline__ bool op_attn_t(Ctx& c, int l, int kvh, int chunk, int q0, bool may_append) {
  CKParams& p = c.p;
  // K/V position steps in flight per lane: 6 for the grouped split-KV
  // instructions (measured best of 4, 6, 8 at KV 4096-32768)
  constexpr int AR = G > 1 ? 6 : ARING;
  constexpr int LPR = HD / 8;     // lanes per K/V row
  constexpr int PPW = 64 / LPR;   // positions per wavefront load
  const int seq = c.seq;
  const int pos = p.start[seq] + c.t;
  const int T = pos + 1;
  const int clen = ((T + p.n_chunks - 1) / p.n_chunks + 15) / 16 * 16;
  const int lo = min(T, chunk * clen), hi = min(T, (chunk + 1) * clen);
  const int hic = min(hi, pos);             // cached positions [lo, hic)
  const bool has_new = lo <= pos && pos < hi;
  const bool append = has_new && may_append;
  const int grp = c.lane / LPR, sub = c.lane % LPR;

  const size_t head_elems = (size_t)p.max_seq * HD;
  uint16_t* const kvs = p.kv + (size_t)seq * p.s_kv;   // this sequence's cache
  const uint16_t* kb = kvs + ((size_t)(l * 2 + 0) * p.hkv + kvh) * head_elems;
  const uint16_t* vb = kvs + ((size_t)(l * 2 + 1) * p.hkv + kvh) * head_elems;
  const uint32_t hbytes = (uint32_t)(head_elems * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kb, hbytes), vr = make_rsrc(vb, hbytes);

  // this wavefront's position blocks: wave, wave + kWaves, ... ; block j covers
  // positions lo + j*PPW + [0, PPW), lane group grp takes one of them
  const int nblk = hic > lo ? (hic - lo + PPW - 1) / PPW : 0;
  const int nsteps = nblk > c.wave ? (nblk - c.wave + kWaves - 1) / kWaves : 0;
  u32x4 rk[AR], rv[AR];
  int pstep = 0;
  // positions past the chunk use an offset beyond the buffer range: the load
  // returns zeros without touching memory, so every issue is unconditional
  auto issue = [&](u32x4& k_, u32x4& v_) {
    const int j = lo + (c.wave + pstep * kWaves) * PPW + grp;
    const int off = j < hic ? (j * HD + sub * 8) * 2 : 0x7ffffff0;
    k_ = __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, kSC1);
    v_ = __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, kSC1);
    ++pstep;
  };
#pragma unroll
  for (int d = 0; d < AR; ++d) issue(rk[d], rv[d]);

  // inputs: raw q of the G heads, k and v of this kv head
  float* qs = c.xs;                 // [G][HD]
  float* ks = c.xs + G * HD;        // [HD]
  float* vs = ks + HD;              // [HD]
  float* wst = vs + HD;             // [kWaves][G][HD + 2] per-wave states
  const uint32_t tag = tag_of(p, c.t, l);
  // this thread's RoPE pair (one of (G + 1) * HD/2 <= kThreads), read before
  // the inputs are waited for
  static_assert((G + 1) * (HD / 2) <= kThreads, "one RoPE pair per thread");
  const int re = c.tid < (G + 1) * (HD / 2) ? c.tid : 0;
  const float cs = ld_f32(p.rope + (size_t)pos * (HD / 2) + re % (HD / 2));
  const float sn = ld_f32(p.rope + (size_t)p.max_seq * (HD / 2) + (size_t)pos * (HD / 2) + re % (HD / 2));
  const uint64_t* qkv = p.qkv + (size_t)seq * p.s_qkv;
  const Fetch f[3] = {{qkv + q0 * HD, G * HD, tag, qs},
                      {qkv + p.qd + kvh * HD, HD, tag, ks},
                      {qkv + p.qd + p.kvd + kvh * HD, HD, tag, vs}};
  // the producers of exactly these words, all three polled together
  // (G * HD <= 512 and HD <= 128 words: one load per thread and input)
  {
    const bool ok = ll_poll_k<3>(c, f);
    (void)ok;   // a stopping wavefront has set the abort word in LDS
    if (!sync_ok(c)) return false;
    mark_ready(c);
  }

  // RoPE (pairs i, i + HD/2) on q heads and k; q pre-scaled for exp2 softmax
  const float qscale = 1.4426950408889634f / sqrtf((float)HD);
  if (c.tid < (G + 1) * (HD / 2)) {
    const int h = c.tid / (HD / 2), i = c.tid % (HD / 2);
    float* x = h < G ? qs + h * HD : ks;
    const float x0 = x[i], x1 = x[i + HD / 2];
    float y0 = x0 * cs - x1 * sn;
    float y1 = x1 * cs + x0 * sn;
    if (h < G) {
      y0 *= qscale;
      y1 *= qscale;
    } else {
      y0 = __uint_as_float(to_bf16(y0) << 16);
      y1 = __uint_as_float(to_bf16(y1) << 16);
    }
    x[i] = y0;
    x[i + HD / 2] = y1;
  }
  for (int i = c.tid; i < HD; i += kThreads) vs[i] = __uint_as_float(to_bf16(vs[i]) << 16);
  __syncthreads();

  // append K and V at pos (the chunk holding pos owns it)
  if (append && c.tid < LPR) {
    u32x4 kw, vw;
    const float* kk = ks + c.tid * 8;
    const float* vv = vs + c.tid * 8;
    kw.x = to_bf16(kk[0]) | (to_bf16(kk[1]) << 16);
    kw.y = to_bf16(kk[2]) | (to_bf16(kk[3]) << 16);
    kw.z = to_bf16(kk[4]) | (to_bf16(kk[5]) << 16);
    kw.w = to_bf16(kk[6]) | (to_bf16(kk[7]) << 16);
    vw.x = to_bf16(vv[0]) | (to_bf16(vv[1]) << 16);
    vw.y = to_bf16(vv[2]) | (to_bf16(vv[3]) << 16);
    vw.z = to_bf16(vv[4]) | (to_bf16(vv[5]) << 16);
    vw.w = to_bf16(vv[6]) | (to_bf16(vv[7]) << 16);
    const int off = (pos * HD + c.tid * 8) * 2;
    __builtin_amdgcn_raw_buffer_store_b128(kw, kr, off, 0, kSC1);
    __builtin_amdgcn_raw_buffer_store_b128(vw, vr, off, 0, kSC1);
  }

  // q slices of this lane
  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) q[g][i] = qs[g * HD + sub * 8 + i];

  AttnState<G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.o[g][i] = 0.f;
  }

  if constexpr (G == 1) {
    // One q head per instruction (the one-chunk mode of short contexts, a
    // few steps per wavefront): the running max is updated per position.
    for (int s0 = 0; s0 < nsteps; s0 += AR) {
#pragma unroll
      for (int d = 0; d < AR; ++d) {
        if (s0 + d < nsteps) {
          const int j = lo + (c.wave + (s0 + d) * kWaves) * PPW + grp;
          const u32x4 kw = rk[d], vw = rv[d];
          float kf[8], vf[8];
          kf[0] = bf_lo(kw.x); kf[1] = bf_hi(kw.x); kf[2] = bf_lo(kw.y); kf[3] = bf_hi(kw.y);
          kf[4] = bf_lo(kw.z); kf[5] = bf_hi(kw.z); kf[6] = bf_lo(kw.w); kf[7] = bf_hi(kw.w);
          vf[0] = bf_lo(vw.x); vf[1] = bf_hi(vw.x); vf[2] = bf_lo(vw.y); vf[3] = bf_hi(vw.y);
          vf[4] = bf_lo(vw.z); vf[5] = bf_hi(vw.z); vf[6] = bf_lo(vw.w); vf[7] = bf_hi(vw.w);
          const bool valid = j < hic;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float sv = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) sv = fmaf(q[g][i], kf[i], sv);
            sv = (LPR == 8) ? sum8(sv) : sum16(sv);
            if (valid) {
              const float M = fmaxf(st.m[g], sv);
              const float a = exp2f(st.m[g] - M), e = exp2f(sv - M);
              st.l[g] = st.l[g] * a + e;
#pragma unroll
              for (int i = 0; i < 8; ++i) st.o[g][i] = fmaf(st.o[g][i], a, e * vf[i]);
              st.m[g] = M;
            }
          }
        }
        issue(rk[d], rv[d]);
      }
    }
  } else {
    // Online softmax one block of AR positions at a time (per lane group):
    // the block's scores first, then one running-max update and one rescale
    // of (l, o) per head, then e = 2^(s - m) and o += e v per position.  Per
    // position that is one exponential and 8 FMAs on o, against two
    // exponentials and a rescale of o when the running max moves per position;
    // at long context attention is bound by this arithmetic.
    for (int s0 = 0; s0 < nsteps; s0 += AR) {
      float sc[AR][G];
  #pragma unroll
      for (int d = 0; d < AR; ++d) {
  #pragma unroll
        for (int g = 0; g < G; ++g) sc[d][g] = -INFINITY;
        if (s0 + d >= nsteps) continue;   // past this wavefront's last step (uniform)
        const int j = lo + (c.wave + (s0 + d) * kWaves) * PPW + grp;
        const bool valid = j < hic;
        const u32x4 kw = rk[d];
        float kf[8];
        kf[0] = bf_lo(kw.x); kf[1] = bf_hi(kw.x); kf[2] = bf_lo(kw.y); kf[3] = bf_hi(kw.y);
        kf[4] = bf_lo(kw.z); kf[5] = bf_hi(kw.z); kf[6] = bf_lo(kw.w); kf[7] = bf_hi(kw.w);
  #pragma unroll
        for (int g = 0; g < G; ++g) {
          float sv = 0.f;
  #pragma unroll
          for (int i = 0; i < 8; ++i) sv = fmaf(q[g][i], kf[i], sv);
          sv = (LPR == 8) ? sum8(sv) : sum16(sv);
          sc[d][g] = valid ? sv : -INFINITY;
        }
      }
  #pragma unroll
      for (int g = 0; g < G; ++g) {
        float M = st.m[g];
  #pragma unroll
        for (int d = 0; d < AR; ++d) M = fmaxf(M, sc[d][g]);
        if (M != -INFINITY) {
          const float a = exp2f(st.m[g] - M);   // 0 while nothing was seen
          st.l[g] *= a;
  #pragma unroll
          for (int i = 0; i < 8; ++i) st.o[g][i] *= a;
          st.m[g] = M;
        }
      }
  #pragma unroll
      for (int d = 0; d < AR; ++d) {
        if (s0 + d < nsteps) {   // uniform
          const u32x4 vw = rv[d];
          float vf[8];
          vf[0] = bf_lo(vw.x); vf[1] = bf_hi(vw.x); vf[2] = bf_lo(vw.y); vf[3] = bf_hi(vw.y);
          vf[4] = bf_lo(vw.z); vf[5] = bf_hi(vw.z); vf[6] = bf_lo(vw.w); vf[7] = bf_hi(vw.w);
  #pragma unroll
          for (int g = 0; g < G; ++g) {
            // an invalid position has score -inf: e = 0 (m is finite once any
            // position of the block was valid; otherwise the block adds nothing)
            const float e = sc[d][g] == -INFINITY ? 0.f : exp2f(sc[d][g] - st.m[g]);
            st.l[g] += e;
  #pragma unroll
            for (int i = 0; i < 8; ++i) st.o[g][i] = fmaf(e, vf[i], st.o[g][i]);
          }
        }
        issue(rk[d], rv[d]);
      }
    }
  }

  // merge the lane groups of this wavefront (xor over group bits)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    float om[G], ol[G], oo[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      om[g] = __shfl_xor(st.m[g], off);
      ol[g] = __shfl_xor(st.l[g], off);
#pragma unroll
      for (int i = 0; i < 8; ++i) oo[g][i] = __shfl_xor(st.o[g][i], off);
    }
    merge_into<G>(st, om, ol, oo);
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float* ws = wst + (c.wave * G + g) * (HD + 2);
      if (sub == 0) { ws[0] = st.m[g]; ws[1] = st.l[g]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) ws[2 + sub * 8 + i] = st.o[g][i];
    }
  }
  // the appended K/V must be visible device-wide before anything that
  // depends on this instruction can run: the storing wavefront waits for its
  // stores to complete before the barrier that precedes the output stores
  if (append && c.wave == 0) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // score of the new position (one per head)
  __syncthreads();
  // (wavefront g < G takes head g: one product per lane, then a wave sum)
  float* pnew = c.red;  // [G] new-position scores
  if (has_new && c.wave < G) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < HD / 64; ++i) s = fmaf(qs[c.wave * HD + i * 64 + c.lane], ks[i * 64 + c.lane], s);
    s = wave_sum(s);
    if (c.lane == 0) pnew[c.wave] = s;
  }
  __syncthreads();

  // final merge over wavefronts (fixed order) and the new position; one
  // thread per (head, element)
  const uint32_t otag = tag;
  for (int e = c.tid; e < G * HD; e += kThreads) {
    const int g = e / HD, i = e % HD;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wst[(w * G + g) * (HD + 2)]);
    if (has_new) M = fmaxf(M, pnew[g]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float* ws = wst + (w * G + g) * (HD + 2);
        const float a = exp2f(ws[0] - M);
        L = fmaf(ws[1], a, L);
        O = fmaf(ws[2 + i], a, O);
      }
      if (has_new) {
        const float a = exp2f(pnew[g] - M);
        L += a;
        O = fmaf(vs[i], a, O);
      }
    }
    const int qh = q0 + g;
    if (p.n_chunks == 1) {
      ll_store(p.aout + (size_t)(qh * HD + i) * c.B + seq, O / L, otag);
    } else {
      uint64_t* pp = p.part + (size_t)seq * p.s_part + ((size_t)qh * p.n_chunks + chunk) * (HD + 2);
      ll_store(pp + 2 + i, O, otag);
      if (i == 0) {
        ll_store(pp + 0, M, otag);
        ll_store(pp + 1, L, otag);
      }
    }
  }
  __syncthreads();
  return true;
}

// One chunk: the instruction is one q head (a), and its kv head's first q
// head appends.  Several chunks: one (kv head a, chunk b) for all its q heads.
template <int HD>
__device__ __forceinline__ bool op_attn_hd(Ctx& c, int l, int a, int b) {
  const int G = c.p.G;
  if (c.p.n_chunks == 1) return op_attn_t<HD, 1>(c, l, a / G, 0, a, a % G == 0);
  switch (G) {
    case 1: return op_attn_t<HD, 1>(c, l, a, b, a, true);
    case 2: return op_attn_t<HD, 2>(c, l, a, b, a * 2, true);
    case 3: return op_attn_t<HD, 3>(c, l, a, b, a * 3, true);
    default: return op_attn_t<HD, 4>(c, l, a, b, a * 4, true);
  }
}

// ---------------------------------------------------------------- opcode: split-KV reduction

// Wavefront 0 turns the chunks' maxima into their weights 2^(m_k - M) (one
// lane per chunk, n <= 64) and the normaliser sum_k l_k 2^(m_k - M); then
// the workgroup's threads split (element, chunk quarter) and add up the
// weighted partial outputs, the quarters in a fixed order.
__device__ __forceinline__ bool op_areduce(Ctx& c, int l, int qh) {
  CKParams& p = c.p;
  const int HD = p.hd, n = p.n_chunks, W = HD + 2;
  const uint32_t tag = tag_of(p, c.t, l);
  // this head's chunk partials, without the attention stage's flags
  // (n * (HD + 2) <= 64 * 130 words: at most 9 loads per thread)
  {
    const bool ok = ll_poll<9>(c, p.part + (size_t)c.seq * p.s_part + (size_t)qh * n * W, n * W, tag, c.xs);
    (void)ok;
    if (!sync_ok(c)) return false;
    mark_ready(c);
  }
  float* const wk = c.red + 128;   // [64] chunk weights, then [4][HD <= 128] quarter sums below
  if (c.wave == 0) {
    const float m = c.lane < n ? c.xs[c.lane * W] : -INFINITY;
    float M = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float a = c.lane < n ? exp2f(m - M) : 0.f;
    const float L = wave_sum(c.lane < n ? c.xs[c.lane * W + 1] * a : 0.f);
    wk[c.lane] = a / L;   // weight of chunk `lane`, normalised
  }
  __syncthreads();
  // thread (quarter q, element i): chunks q, q + 4, ...
  float* const qs = c.xs + n * W;   // [4][HD] quarter sums, after the partials
  if (c.tid < 4 * HD) {
    const int q = c.tid / HD, i = c.tid - q * HD;
    float O = 0.f;
    for (int k = q; k < n; k += 4) O = fmaf(c.xs[k * W + 2 + i], wk[k], O);
    qs[q * HD + i] = O;
  }
  __syncthreads();
  for (int i = c.tid; i < HD; i += kThreads)
    ll_store(p.aout + (size_t)(qh * HD + i) * c.B + c.seq,
             (qs[i] + qs[HD + i]) + (qs[2 * HD + i] + qs[3 * HD + i]), tag);
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------- the kernel

static __shared__ int s_flags[8];

// The persistent loop.  Three kernels instantiate it: dense models with one
// sequence (batch size the constant 1), MoE models with one sequence, and
// dense models with several sequences (batch size from the parameters).  No
// kernel carries the others' code: the register allocation and code layout
// of each stay its own (the batched GEMV in the batch-1 kernel cost it 4%;
// a change to the MoE opcodes alone moved it by 2%).
enum KernelKind { K_DENSE = 0, K_MOE = 1, K_BATCH = 2 };
template <int KIND>
__device__ __forceinline__ void megakernel_body() {
  constexpr bool BATCHED = KIND == K_BATCH, MOE = KIND == K_MOE;
  // The parameters are read in place in the kernel-argument segment (they
  // are the first and only argument): referring to the by-value parameter
  // itself would make the compiler copy it to scratch memory.
  CKParams* pk = (CKParams*)__builtin_amdgcn_kernarg_segment_ptr();
  extern __shared__ __align__(16) float smem[];
  lds_vint* sflag = (lds_vint*)s_flags;
  const int wg = blockIdx.x;
  if (threadIdx.x == 0) {
    sflag[0] = 0;
    sflag[1] = 0;
    sflag[2] = -1;
    sflag[kPredStamp] = -1;
    ((int*)(smem + pk->x_floats + pk->res_floats + pk->out_floats))[kSpecHitWord] = 0;
    ((int*)(smem + pk->x_floats + pk->res_floats + pk->out_floats))[kSpecNWord] = 0;
    if constexpr (MOE) ((int*)(smem + pk->x_floats + pk->res_floats + pk->out_floats))[kRouteStamp] = 0;
  }
  __syncthreads();
  const int n = ldc_i32(pk->sched + kWords + wg);
  bool ok = true;
  for (int t = 0; t < pk->n_steps && ok; ++t) {
    // Workgroup 0 reads the stop word once per step, between its last
    // instruction of the previous step and the wait for this step's inputs
    // (which the other workgroups' last tiles keep open): waits that end
    // sooner than the pollers' stop checks cannot hide a stop request.  Once
    // it stops publishing, every other workgroup ends up waiting on it long
    // enough to see the abort word.
    if (wg == 0 && __hip_atomic_load(pk->stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) {
      if (threadIdx.x == 0) raise_at(pk->status, sflag, MKD_E_ABORTED, true, wg, 0, t);
      ok = false;
      break;
    }
    for (int i = 0; i < n && ok; ++i) {
      // Opaque copies of the parameter pointer and thread id: nothing that
      // depends on them is hoisted out of the persistent loop, so values one
      // opcode needs do not stay live (and spill) through all the others.
      CKParams* pp = pk;
      int tid = threadIdx.x;
      asm volatile("" : "+s"(pp));
      asm volatile("" : "+v"(tid));
      CKParams& p = *pp;
      const int32_t* ins = p.sched + kWords + p.n_wg + ((size_t)wg * p.max_instr + i) * kWords;
      const int op = ldc_i32(ins + I_OP), l = ldc_i32(ins + I_LAYER), a = ldc_i32(ins + I_A),
                b = ldc_i32(ins + I_B), index = ldc_i32(ins + I_INDEX);
      uint64_t* tr = p.trace ? p.trace + (((size_t)wg * p.n_steps + t) * p.max_instr + i) * kTraceWords
                             : nullptr;
      Ctx c{p, smem, smem + p.x_floats, smem + p.x_floats + p.res_floats,
            smem + p.x_floats + p.res_floats + p.out_floats,
            sflag, wg, i, t, tid, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6),
            ldc_i32(ins + I_STAGE), index, tr, BATCHED ? ldc_i32(ins + I_SEQ) : 0, BATCHED ? p.B : 1};
      if (tr && tid == 0) st_u64(tr, wall_clock64());
      // The first weight units of the next dense gate/up instruction are
      // staged in LDS by this one: at the start of an O-projection (whose
      // wait spans the whole attention phase), else at the end of the
      // instruction, once its own loads are done.
      const int32_t* nx = i + 1 < n ? ins + kWords : nullptr;
      const int nxop = nx ? ldc_i32(nx + I_OP) : OP_NOP;
      const bool stage = !MOE && p.pre_units > 0 && nxop == OP_UPGATE;
      // MoE with the expert prediction on: O-projection tile 0 first predicts
      // and publishes the layer's experts, and an O-projection followed by a
      // gate/up tile fetches them
      const bool predict = MOE && p.predict && op == OP_OPROJ;
      if (stage && op == OP_OPROJ) {
        if constexpr (BATCHED) stage_upgate_b(c, ldc_i32(nx + I_LAYER), ldc_i32(nx + I_A), ldc_i32(nx + I_B));
        else stage_upgate(c, ldc_i32(nx + I_LAYER), ldc_i32(nx + I_A), ldc_i32(nx + I_B));
      }
      if constexpr (MOE) {
        if (predict && index == 0) ok = predict_publish(c, l);
      }
      if (ok) switch (op) {
        case OP_QKV:
        case OP_OPROJ:
        case OP_UPGATE:
        case OP_DOWN:
        case OP_LMHEAD:
          ok = op_gemv_any<BATCHED>(c, op, l, a, b, index, predict && nxop == OP_MOE_UPGATE);
          break;
        case OP_ATTN: ok = p.hd == 64 ? op_attn_hd<64>(c, l, a, b) : op_attn_hd<128>(c, l, a, b); break;
        case OP_AREDUCE: ok = op_areduce(c, l, a); break;
        case OP_MOE_UPGATE:
          if constexpr (MOE) ok = op_moe_upgate(c, l, a, b, index);
          break;
        case OP_MOE_DOWN:
          if constexpr (MOE) ok = op_moe_down(c, l, a, b);
          break;
        default: break;
      }
      if (ok) signal_done(c);
      if (ok && stage && op != OP_OPROJ) {
        if constexpr (BATCHED) stage_upgate_b(c, ldc_i32(nx + I_LAYER), ldc_i32(nx + I_A), ldc_i32(nx + I_B));
        else stage_upgate(c, ldc_i32(nx + I_LAYER), ldc_i32(nx + I_A), ldc_i32(nx + I_B));
      }
    }
  }
  if constexpr (MOE) {
    // this workgroup's expert-prediction counts, summed over workgroups
    if (pk->predict && threadIdx.x == 0) {
      const int* cnt = (const int*)(smem + pk->x_floats + pk->res_floats + pk->out_floats);
      atomicAdd(pk->status + S_SPEC_HIT, cnt[kSpecHitWord]);
      atomicAdd(pk->status + S_SPEC_N, cnt[kSpecNWord]);
    }
  }
  // the last step's argmax
  if (ok && wg == 0) {
    CKParams& p = *pk;
    const int tid = threadIdx.x;
    Ctx c{p, smem, smem + p.x_floats, smem + p.x_floats + p.res_floats,
          smem + p.x_floats + p.res_floats + p.out_floats,
          sflag, wg, 0, p.n_steps, tid, tid & 63, __builtin_amdgcn_readfirstlane(tid >> 6), 0, 0,
          nullptr, 0, BATCHED ? p.B : 1};
    if (fetch_partials(c, p.n_steps - 1)) {
      for (int b = 0; b < c.B; ++b) {
        const int am = argmax_staged(c, b);
        if (tid == 0) st_i32(p.tokens_out + (size_t)b * p.n_steps + p.n_steps - 1, am);
      }
    }
  }
}

}  // namespace mkd
