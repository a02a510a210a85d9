// moe_kernels.hip -- the MoE-layer forward for gfx950 (MI355X), behind the C ABI of moe.h.
//
// One persistent kernel runs the whole layer.  Its work items are pulled from atomic ticket
// counters in the workspace (the global task queue with an atomic counter of the Weave
// review, section 2.2; the work-conserving tile scheduler of the FlashMoE explainer,
// section 四), one counter per partition of the workgroups, in this order:
//
//   Z  clear the per-m-tile dependency counters (and chunk histograms)
//   L  router logits (MFMA): 16 tokens x 16 experts per item, K split over the 4 waves, or
//      on the expert tile core 16-64 tokens x 128-256 experts over a part of K
//      (Z and L take no ticket: each workgroup runs its share of them first)
//   K  top-k + softmax over the kept logits for a group of tokens; the last K item to
//      finish builds the plan (expert offsets, the m-tile descriptor table) and, for a
//      batch that is one scatter chunk, scatters it
//   SG shared-expert gate/up items (need no routing, so they overlap the routing)
//   Q  fp8 activations only: quantise 16 hidden rows to E4M3 with per-block scales
//   S  stable scatter of a chunk: perm / inv_perm (batches of several chunks)
//   G  gate/up items (m-tile, H columns): gathered token rows x W_gate/W_up, SwiGLU in
//      registers, H written once
//   D  down items (m-tile, output columns): H rows x W_down -> Y
//   C  combine items: out[t] = sum_j w[t,j] * Y[inv_perm[t*k+j]] (+ Y_shared[t]), fixed
//      slot order, summed in float32 and rounded once to the output, no float atomics (H and Y
//      themselves are stored in the activation dtype)
//
// A work item only ever waits for items earlier in this order.  Ticketed items were taken
// by workgroups that are running (a workgroup holds at most its current ticket and the next
// one it prefetched, which is larger; a gate/up or down item's completion counter left
// pending at its end is incremented before the workgroup waits for anything); the Z and L items, which wait for nothing, are bound
// to workgroups, and the launch never has more workgroups than can be resident at once, so
// each of those runs too.  So every wait ends, whatever the grid size.  Every wait is also
// bounded in time; a timeout sets a fault flag that makes every later wait give up, so the
// kernel always exits.
//
// Expert tiles: weights are the MFMA A operand (rows = output channels, in a packed
// fragment layout, one 16-byte load per lane straight from HBM into registers), token rows
// are the B operand.  This is the operand-swapped form that suits small M (GC-MoE article,
// "two MMA implementations"): the weight stream, the HBM-bound part, is read once per item
// and never passes through LDS.  Decode-sized m-tiles (16 rows) read the token rows
// straight into registers; larger m-tiles stage them in LDS with the load-to-LDS path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"
#include "moe_plan.h"

namespace {

using namespace moe;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// 16-byte streaming (nontemporal) load from global memory; the explicit address space keeps
// it a global_load even when the address comes from a select with a uniform value
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)p));
}

// kernel kinds: weight dtype, and for fp8 weights whether the GEMMs read fp8 activations
// (WQ8: E4M3 activations with power-of-two block scales, fp8 matrix cores; m-tiles > 16 rows)
enum : int { WF32 = 0, WBF16 = 1, WFP8 = 2, WQ8 = 3 };
constexpr bool is_fp8w(int wt) { return wt == WFP8 || wt == WQ8; }

constexpr int kCpolNt = 2;  // cache policy of a buffer load: nontemporal (streamed once)

// KU: K elements per 16-byte weight load of one lane; WSZ/ASZ: weight/activation bytes
template <int WT> struct Ty;
template <> struct Ty<WF32> { static constexpr int KU = 16, WSZ = 4, ASZ = 4; };
template <> struct Ty<WBF16> { static constexpr int KU = 32, WSZ = 2, ASZ = 2; };
template <> struct Ty<WFP8> { static constexpr int KU = 64, WSZ = 1, ASZ = 2; };
template <> struct Ty<WQ8> { static constexpr int KU = 64, WSZ = 1, ASZ = 1; };

// per-kernel tile shape: MG 16-token groups per m-tile, NF weight fragments per wave,
// FL 16-byte weight loads per fragment per K chunk
#ifndef MOE_FP8_FOLD_MG
#define MOE_FP8_FOLD_MG 4
#endif
template <int WT, int MG> struct Shape {
  static constexpr int NF = MG == 1 ? 2 : 4;
  // register/LDS buffers: three (two K chunks in flight) where registers and LDS allow it,
  // else two (one chunk in flight): the 32-row fp8 tiles (registers) and the 160-row fp8
  // tiles (three 40 KB activation stages and the routing scratch exceed the 160 KB of LDS)
#ifndef MOE_NBUF
#define MOE_NBUF(WT, MG) ((WT == WFP8 && (MG == 2 || MG == 10)) ? 2 : 3)
#define MOE_FL(WT, MG) ((WT != WFP8 && MG == 1) ? 4 : 2)
#endif
  static constexpr int NBUF = MOE_NBUF(WT, MG);
  static constexpr int FL = MOE_FL(WT, MG);
};

struct KParams {
  int T, d, n, E, k, S;
  int phases;
  int bm, tk, gu_cols, dn_cols;
  int n_lt, n_le, n_kt, n_kc, n_shmt, nt_gu, nt_dn, n_comb, mt_cap;
  int kt_tok;                     // tokens per top-k item
  int ctok;       // tokens per combine item
  int n_Z, n_L, n_K, n_SG, n_S;   // items per static phase (order Z, L, K, SG, S)
  int gd_words, hist_words;       // words cleared by the Z items
  int schedule;  // 0 dynamic, 1 static
  int reset_err;  // 1: the last workgroup out also clears the fault flag (fixed scratch, whose
                  //    flag no caller can read)
  int late;       // 1: gate/up and down items from the per-XCD queues, grouped order (see the kernel)
  int group_m;    // late phase: m-tiles per group
  int aq;         // 1: fp8 activations (Q items quantise the hidden rows; H is requantised)
  int n_Q;        // activation-quantisation items (ticketed, before the scatter items)
  int xs_stride, hs_stride;  // bytes per row of the hidden / H block-scale arrays
  const void *x, *wr;
  const float *bias;
  const void *wg, *wu, *wd;
  const float *sg, *su, *sd;
  const void *shg, *shu, *shd;
  const float *shsg, *shsu, *shsd;
  void *out;
  float *logits;
  int *ids;
  float *wts;
  int *counts, *offsets, *perm, *inv_perm;
  int *ctrl, *gudone, *hist, *mtoff;
  int *mtok;      // 16-row m-tiles: token of each row, m-tile-major (rows past the end: stale)
  int *dndone;    // per m-tile (shared first): down items done
  int rt_split;   // K splits per router tile; > 1: partial logits in lpart [rt_split][T][E]
  float *lpart;
  int *slotmt;    // [T*k] routed m-tile of each (token, slot)
  int4 *desc;
  void *H, *Y;
  uint8_t *xq;    // fp8 activations: E4M3 codes of the hidden rows [T][d]
  uint8_t *xs;    // ... their block scales, 2^(xs - 127) per 128-wide block [T][xs_stride]
  uint8_t *hs;    // ... block scales of H (H itself then holds E4M3 codes) [rows][hs_stride]
  unsigned long long *trace;
  long long trace_cap;
};

// work item kinds (trace records)
enum ItemKind : int {
  K_ZERO = 0, K_ROUTER = 1, K_TOPK = 2, K_SHGU = 3, K_SCATTER = 4, K_GU = 5, K_DN = 6, K_COMB = 7, K_QUANT = 8
};

// ---------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  return (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v) |
         ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32)) << 32);
}

// otid() behind an empty volatile asm: values derived from it are recomputed in each
// work item instead of being hoisted out of the persistent loop (where they would stay
// live, in registers, across every item)
// p, passed through an empty volatile asm: what it points to is unknown to the compiler
// afterwards, so loads through it stay ordered with memory-clobbering asm statements
__device__ __forceinline__ const char *laundered(const char *p) {
  asm volatile("" : "+v"(p));
  return p;
}

// Expert weights are in the packed fragment layout: the 16 rows of a fragment are stored K
// step by K step, each step (64 bytes of each row) one contiguous 1 KB block in MFMA lane
// order, so lane l's 16 bytes of step s sit at fragment + s * kWStep + 16 * l.  A fragment
// spans the same bytes as its 16 rows in row-major order (it starts at row r0's offset).
constexpr int kWStep = 1024;
__device__ __forceinline__ const char *frag_ptr(const void *mat, int r0, size_t rb, int lane) {
  return reinterpret_cast<const char *>(mat) + (size_t)r0 * rb + lane * 16;
}

__device__ __forceinline__ int otid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima): at most N vector memory
// operations of this wave still outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");  // memory accesses stay on their side of the wait
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_vm0() { wait_vm<0>(); }

// Workgroup barrier without the fences of __syncthreads.  Those fences wait for every
// outstanding vector memory operation (the LDS DMA counts as one), which would drain the
// prefetch pipeline at every K chunk.  The caller has already waited for the LDS data the
// barrier publishes; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The activation staging buffers are three separate LDS variables: the compiler can then
// tell that a read of one buffer does not depend on a DMA still filling another, and does
// not wait for the prefetches before every LDS read.
struct Lds3 {
  char *b0, *b1, *b2, *b3;  // (b3: four-stage kernels only)
  uint8_t *sl;              // fp8 activations: block scales of the tile's rows (WQ8 kernels only)
};

__device__ __forceinline__ char *stage_buf(const Lds3 &lb, int st) {
  return st == 0 ? lb.b0 : st == 1 ? lb.b1 : st == 2 ? lb.b2 : lb.b3;
}

// 16 bytes per lane, global -> LDS, as a buffer load: lane l reads base + voff (its own
// offset) + soff (uniform) and lands at lds_base + 16*l (lds_base uniform).  COH selects the
// device-coherent cache policy (SC1) for data written in this launch.  The compiler counts
// these loads like any other (its vmcnt waits stay exact) and, with the stage buffers as
// separate LDS variables, makes an LDS read wait only for loads into the buffer it reads;
// with the offsets in loop-invariant and scalar registers, no vector register is rewritten
// per stage.
constexpr int kCpolSc1 = 16;  // cache policy: device-coherent (SC1)
template <bool COH>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, void *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_base, 16, voff, soff, 0,
                                           COH ? kCpolSc1 : 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
}

// Load through a wave-uniform pointer to data that is read-only for the whole launch (the
// weight block scales): a scalar load, counted apart from the vector memory operations, so
// waiting for it never waits for the tile pipeline's prefetches
__device__ __forceinline__ float ld_uniform(const float *p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) float *>(uni64(reinterpret_cast<uint64_t>(p)));
}

__device__ __forceinline__ int ld_relaxed(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Data that one workgroup writes and another reads during the same launch moves through
// device-coherent accesses (agent-scope relaxed atomics: stores write through to the
// device coherence point, loads never hit a stale line of another XCD's L2).  A producer
// then only waits for its stores to complete (s_waitcnt) before bumping a counter, and a
// consumer reads after seeing the counter: no agent-scope fence, so no whole-L2 write-back
// or invalidation on the hot path (those cost more than the work items themselves).
// (every pointer is cast to the global address space: the data always lives in device
// memory, and a generic pointer would make these flat accesses, which the compiler has to
// wait for conservatively)
typedef __attribute__((address_space(1))) int gint;
typedef __attribute__((address_space(1))) uint64_t gu64;
__device__ __forceinline__ void st_coh(int *p, int v) { __hip_atomic_store((gint *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_coh(float *p, float v) {
  __hip_atomic_store((gint *)p, __float_as_int(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(void *p, uint64_t v) {
  __hip_atomic_store((gu64 *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
typedef __attribute__((address_space(1))) uint8_t gu8;
__device__ __forceinline__ void st_coh8(void *p, uint32_t v) {
  __hip_atomic_store((gu8 *)p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_coh(const int *p) {
  return __hip_atomic_load((const gint *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float *p) {
  return __int_as_float(__hip_atomic_load((const gint *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint64_t ld_coh64(const void *p) {
  return __hip_atomic_load((const gu64 *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// plain 16-byte global load (data not written during this launch)
__device__ __forceinline__ uint4 ld_glob16(const void *p) {
  return __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4 *)p);
}
__device__ __forceinline__ int4 ld_coh_int4(const int4 *p) {
  const uint64_t a = ld_coh64(p), b = ld_coh64(reinterpret_cast<const char *>(p) + 8);
  return make_int4((int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)(uint32_t)b, (int)(uint32_t)(b >> 32));
}
__device__ __forceinline__ uint4 ld_coh16(const void *p) {
  const uint64_t a = ld_coh64(p), b = ld_coh64(reinterpret_cast<const char *>(p) + 8);
  return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}
__device__ __forceinline__ void st_coh_int4(int4 *p, int4 v) {
  st_coh64(p, (uint64_t)(uint32_t)v.x | ((uint64_t)(uint32_t)v.y << 32));
  st_coh64(reinterpret_cast<char *>(p) + 8, (uint64_t)(uint32_t)v.z | ((uint64_t)(uint32_t)v.w << 32));
}

constexpr uint64_t kSpinTicks = 200000000ull;  // ~2 s of the 100 MHz wall clock

// Thread 0 only: wait until *p >= target.  False on timeout or an earlier fault.
// Polls with relaxed agent-scope loads (an acquire load would invalidate caches on every
// poll).  No fence follows a successful wait: everything the waiter then reads that another
// workgroup wrote in this launch is read with device-coherent loads (sc1, past this XCD's
// L2), and the producer's data stores had completed (s_waitcnt vmcnt(0)) before its counter
// increment was issued, so the data is at the coherence point before the counter.  Polls back off
// from ~0.1 us to ~0.9 us apart: hundreds of waiting workgroups polling one address at full
// rate would saturate that address's memory channel and slow every other load.
// spin_value returns the value it saw (>= target >= 0), or -1 on timeout or fault.
// fast: polls stay ~0.1 us apart (for waits of a few workgroups at the end of the layer).
__device__ __forceinline__ int spin_value(const int *p, int target, int *err, bool fast = false) {
  int v = ld_relaxed(p);
  if (v >= target) return v;
  const uint64_t t0 = wall_clock64();
  for (int it = 0;; ++it) {
    if (fast || it < 8) __builtin_amdgcn_s_sleep(4);
    else if (it < 32) __builtin_amdgcn_s_sleep(12);
    else __builtin_amdgcn_s_sleep(32);
    v = ld_relaxed(p);
    if (v >= target) return v;
    if (ld_relaxed(err) != 0) return -1;
    if (wall_clock64() - t0 > kSpinTicks) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return -1;
    }
  }
}
__device__ __forceinline__ bool spin_geq(const int *p, int target, int *err, bool fast = false) {
  return spin_value(p, target, err, fast) >= 0;
}

__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  // exact for values with <= 8 significant bits (decoded fp8 values)
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// 8 OCP e4m3 codes -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t a, uint32_t b) {
  const f2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, false);
  const f2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, true);
  const f2v p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
  const f2v p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);
  uint4 r;
  r.x = pack_hi16(p0.x, p0.y);
  r.y = pack_hi16(p1.x, p1.y);
  r.z = pack_hi16(p2.x, p2.y);
  r.w = pack_hi16(p3.x, p3.y);
  return __builtin_bit_cast(bf16x8, r);
}

// 8 OCP e4m3 codes times a block scale -> 8 bf16: each decoded value (exact in fp32) is
// multiplied by the scale in fp32 and the product rounded to bf16, nearest even (the hardware's
// scaled conversions take only the scale's exponent, so the multiply is explicit)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16_scaled(uint32_t a, uint32_t b, float s) {
  const f2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, false);
  const f2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, true);
  const f2v p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
  const f2v p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);
  return bf16x8{static_cast<__bf16>(p0.x * s), static_cast<__bf16>(p0.y * s), static_cast<__bf16>(p1.x * s),
                static_cast<__bf16>(p1.y * s), static_cast<__bf16>(p2.x * s), static_cast<__bf16>(p2.y * s),
                static_cast<__bf16>(p3.x * s), static_cast<__bf16>(p3.y * s)};
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// silu(g) * u = g / (1 + e^-g) * u, the quotient by the hardware reciprocal (about 1 ulp of
// float32, far below the rounding of H to the activation dtype; an IEEE division costs a
// dozen vector instructions, 80 of them per lane at the end of a 160-row gate/up item)
__device__ __forceinline__ float silu_mul(float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; }

// monotone map float -> uint32 (after -0.0 -> +0.0): larger float -> larger key
__device__ __forceinline__ uint32_t ordered_key(float v) {
  v = v + 0.0f;  // -0.0 + 0.0 = +0.0 under round-to-nearest
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// one MFMA step: acc += W(16 rows x KU) . A(16 tokens x KU)^T over this lane's K slice
template <int WT>
__device__ __forceinline__ f4 mfma_step(const uint4 &w, const uint4 &a0, const uint4 &a1, f4 acc) {
  if constexpr (WT == WBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, a0),
                                                   acc, 0, 0, 0);
  } else if constexpr (WT == WF32) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), __uint_as_float(a0.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), __uint_as_float(a0.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), __uint_as_float(a0.z), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), __uint_as_float(a0.w), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w.x, w.y), __builtin_bit_cast(bf16x8, a0), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w.z, w.w), __builtin_bit_cast(bf16x8, a1), acc, 0, 0, 0);
  }
}

// One fp8 x fp8 MFMA over a 128-wide K block (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x
// E4M3): lane (g, j) gives the 32 codes of weight row j and of token j at the same K
// positions (its two 16-byte halves: K [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of
// the block), and the token's block scale as an 8-bit exponent (2^(sb - 127)); the weight
// side's scale is 1 (exponent 127).  Lane (g, j)'s exponent scales 32 of the K terms of
// token j, and the four lanes of a token hold the same one, so all 128 terms carry it.
__device__ __forceinline__ f4 mfma_fp8x8(const uint4 &w0, const uint4 &w1, const uint4 &a0, const uint4 &a1, int sb) {
  const v8i A = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
  const v8i B = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, sb);
}

// Block scale of fp8 activations: the smallest s >= -127 with amax <= 448 * 2^s, from the bits
// of amax = (1 + M / 2^23) * 2^(E - 127): 448 * 2^s = 1.75 * 2^(s + 8), so s = E - 135 when
// M <= 0.75 * 2^23, else E - 134 (exact; zero and subnormal amax give -127)
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int s = (int)(u >> 23) - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return s > -127 ? s : -127;
}

// 4 floats times 2^-s -> 4 E4M3 codes (round to nearest even; |v| * 2^-s <= 448 by the choice
// of s), packed little-endian
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, int s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(a, -s), __builtin_ldexpf(b, -s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(c, -s), __builtin_ldexpf(d, -s), w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------------
// expert tile core: acc[NF][MG] = W[NF frags of 16 rows, K] . A[MG groups of 16 rows, K]^T
//
// lane l = 16*g + j holds weight row (frag base + j), bytes [64*f + 16*g, +16) of every
// 64-byte step f of the row, and the activation operand of token (16*mg + j) over the
// same K positions; result D[4*g + r][j] = channel (frag base + 4*g + r), token 16*mg + j.
// ---------------------------------------------------------------------------------
// Branch-free token groups: the small tiles and the fp8-activation tiles (their block-scaled
// products then pipeline with the MFMAs; 20 % faster).  The larger bf16, fp32 and w8a16 tiles
// skip absent groups (computing them cost more on partly filled m-tiles: skewed layer 829 ->
// 972 us with every group computed).
template <int WT, int MG> struct Core {
  static constexpr int NF = Shape<WT, MG>::NF, FL = Shape<WT, MG>::FL;
  static constexpr int KU = Ty<WT>::KU, ASZ = Ty<WT>::ASZ;
  static constexpr int KC = FL * KU;            // K per chunk
  static constexpr int RB = KC * ASZ;           // activation bytes per row per chunk
  static constexpr int NCOL = RB / 16;          // 16-byte columns per row
  static constexpr int BMR = MG * 16;
  static constexpr int RPK = 1024 / RB;         // rows per 1 KB load-to-LDS block
  static constexpr int NKB = BMR * RB / 1024;             // 1 KB load-to-LDS blocks per chunk
  static constexpr int NDMA = NKB >= kWaves ? NKB / kWaves : 1;  // per wave (waves >= NKB: none)
  static constexpr int BUF = BMR * RB;          // bytes of one LDS buffer
  static constexpr int NBUF = Shape<WT, MG>::NBUF;
  static constexpr int PER_CHUNK = NDMA + NF * FL;  // vector memory ops per wave per chunk
  static_assert(NKB >= 1 && RPK >= 1 && (NKB < kWaves || NKB % kWaves == 0), "tile shape");

  // the MFMAs of one K chunk; FULL: every token group is present (no per-group branch,
  // so LDS reads and MFMAs of different groups interleave freely)
  template <bool FULL>
  __device__ static __forceinline__ void chunk_mfma(f4 (&acc)[NF][MG], const uint4 (&W)[NF][FL], const char *A,
                                                    const float *const (&sc)[NF], int c, int ngroups, int g, int j,
                                                    const uint8_t *SL, int sstride) {
    if constexpr (WT == WQ8) {
      // one 128-wide K block per chunk: per token group, the two 16-byte halves of each row's
      // codes and the row's block exponent, read from LDS LA groups ahead of their MFMAs; the
      // block's products are scaled by the weight block scale into the accumulators
      static_assert(FL == 2, "one scale block per chunk");
      constexpr int LA = MG < 2 ? MG : 2;
      struct Bop {
        uint4 lo, hi;
        int s;
      };
      auto rd = [&](int b) {
        const int r = b * 16 + j;
        Bop o;
        o.lo = *reinterpret_cast<const uint4 *>(A + r * RB + ((g ^ (r & (NCOL - 1))) << 4));
        o.hi = *reinterpret_cast<const uint4 *>(A + r * RB + (((g + 4) ^ (r & (NCOL - 1))) << 4));
        o.s = SL[r * sstride + c];
        return o;
      };
      float sw[NF];
#pragma unroll
      for (int a = 0; a < NF; ++a) sw[a] = ld_uniform(sc[a] + c);
      Bop bv[LA];
#pragma unroll
      for (int t = 0; t < LA; ++t) bv[t] = rd(t);
      f4 prev;  // the last product not yet scaled into its accumulators
#pragma unroll
      for (int b = 0; b < MG; ++b) {
        const Bop cur = bv[b % LA];
        if (b + LA < MG) bv[b % LA] = rd(b + LA);
        if (FULL || b == 0 || b < ngroups) {
          // each product is scaled into its accumulators after the next MFMA is issued, so
          // that the vector FMAs overlap an MFMA instead of waiting for their own (with one
          // result register for every product, each MFMA would wait for the previous FMAs);
          // the present groups are a prefix, so group b - 1's last product is still pending
          // here unless b is the first group, and the last present group scales its own
          f4 r = mfma_fp8x8(W[0][0], W[0][1], cur.lo, cur.hi, cur.s);
          if (b > 0) acc[NF - 1][b - 1] += prev * sw[NF - 1];
          prev = r;
#pragma unroll
          for (int a = 1; a < NF; ++a) {
            r = mfma_fp8x8(W[a][0], W[a][1], cur.lo, cur.hi, cur.s);
            acc[a - 1][b] += prev * sw[a - 1];
            prev = r;
          }
          if (b + 1 == MG || !(FULL || b + 1 < ngroups)) acc[NF - 1][b] += prev * sw[NF - 1];
        }
      }
    } else if constexpr (WT == WFP8 && MG >= MOE_FP8_FOLD_MG) {
      // fp8 weights, scale folded: the 16 rows of a fragment lie in one 128-row scale block, so
      // each fragment has one block scale per 128-wide K block; its codes are decoded, multiplied
      // by that scale and rounded to bf16 once per chunk, shared by the MG token groups, and the
      // MFMAs accumulate straight into acc (no per-block partial sums to scale)
      // (FL == 1: a chunk is half of a 128-wide scale block, chunk c in block c / 2)
      constexpr int SPB = FL < 2 ? 1 : 2;  // steps per scale block within a chunk
      constexpr int BPC = FL / SPB;        // scale blocks per chunk (a step is 64 codes)
      bf16x8 D[NF][FL][2];
#pragma unroll
      for (int blk = 0; blk < BPC; ++blk) {
#pragma unroll
        for (int a = 0; a < NF; ++a) {
          const float s = ld_uniform(sc[a] + (FL < 2 ? (c >> 1) : c * BPC + blk));
#pragma unroll
          for (int ff = 0; ff < SPB; ++ff) {
            const uint4 &w = W[a][blk * SPB + ff];
            D[a][blk * SPB + ff][0] = fp8x8_to_bf16_scaled(w.x, w.y, s);
            D[a][blk * SPB + ff][1] = fp8x8_to_bf16_scaled(w.z, w.w, s);
          }
        }
      }
      // the activation operands of the FL * MG (step, group) pairs, LA pairs ahead of their
      // MFMAs; a step's 64 K positions of this lane are two 16-byte columns of the row
      constexpr int NP = FL * MG, LA = NP < 3 ? NP : 3;
      struct Aop {
        uint4 a0, a1;
      };
      auto rd = [&](int t) {
        const int f = t / MG, b = t % MG, r = b * 16 + j, c0 = f * 8 + 2 * g;
        Aop o;
        o.a0 = *reinterpret_cast<const uint4 *>(A + r * RB + ((c0 ^ (r & (NCOL - 1))) << 4));
        o.a1 = *reinterpret_cast<const uint4 *>(A + r * RB + (((c0 + 1) ^ (r & (NCOL - 1))) << 4));
        return o;
      };
      Aop av[LA];
#pragma unroll
      for (int t = 0; t < LA; ++t) av[t] = rd(t);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const int f = t / MG, b = t % MG;
        const Aop cur = av[t % LA];
        if (t + LA < NP) av[t % LA] = rd(t + LA);
        if (FULL || b == 0 || b < ngroups) {
#pragma unroll
          for (int a = 0; a < NF; ++a) {
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(D[a][f][0], __builtin_bit_cast(bf16x8, cur.a0), acc[a][b], 0, 0, 0);
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(D[a][f][1], __builtin_bit_cast(bf16x8, cur.a1), acc[a][b], 0, 0, 0);
          }
        }
      }
    } else if constexpr (WT == WFP8) {
      constexpr int BPC = FL / 2;             // 128-wide scale blocks per chunk
      constexpr int MGC = MG < 4 ? MG : 4;    // token groups per partial-sum pass
#pragma unroll
      for (int blk = 0; blk < BPC; ++blk) {
        float s[NF];
#pragma unroll
        for (int a = 0; a < NF; ++a) s[a] = ld_uniform(sc[a] + c * BPC + blk);
#pragma unroll
        for (int b0 = 0; b0 < MG; b0 += MGC) {
          if (FULL || b0 == 0 || b0 < ngroups) {
            f4 tmp[NF][MGC];
#pragma unroll
            for (int a = 0; a < NF; ++a)
#pragma unroll
              for (int b = 0; b < MGC; ++b) tmp[a][b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ff = 0; ff < 2; ++ff) {
              const int f = blk * 2 + ff;
#pragma unroll
              for (int b = 0; b < MGC; ++b) {
                if (FULL || b0 + b == 0 || b0 + b < ngroups) {
                  const int r = (b0 + b) * 16 + j;
                  const int c0 = f * 8 + 2 * g;
                  const uint4 a0 = *reinterpret_cast<const uint4 *>(A + r * RB + ((c0 ^ (r & (NCOL - 1))) << 4));
                  const uint4 a1 = *reinterpret_cast<const uint4 *>(A + r * RB + (((c0 + 1) ^ (r & (NCOL - 1))) << 4));
#pragma unroll
                  for (int a = 0; a < NF; ++a) tmp[a][b] = mfma_step<WT>(W[a][f], a0, a1, tmp[a][b]);
                }
              }
            }
#pragma unroll
            for (int a = 0; a < NF; ++a)
#pragma unroll
              for (int b = 0; b < MGC; ++b) acc[a][b0 + b] += tmp[a][b] * s[a];
          }
        }
      }
    } else {
      // the activation operands of the FL * MG (step, group) pairs, read from LDS LA pairs
      // ahead of their MFMAs (an LDS read consumed at once would expose its latency before
      // every group's four MFMAs); every read is unconditional (rows past the tile's end
      // repeat its last row), only the MFMAs of absent groups are skipped
      constexpr int NP = FL * MG, LA = NP < 3 ? NP : 3;
      auto rd = [&](int t) {
        const int f = t / MG, b = t % MG, r = b * 16 + j, c0 = f * 4 + g;
        return *reinterpret_cast<const uint4 *>(A + r * RB + ((c0 ^ (r & (NCOL - 1))) << 4));
      };
      uint4 av[LA];
#pragma unroll
      for (int t = 0; t < LA; ++t) av[t] = rd(t);
#pragma unroll
      for (int t = 0; t < NP; ++t) {
        const int f = t / MG, b = t % MG;
        const uint4 cur = av[t % LA];
        if (t + LA < NP) av[t % LA] = rd(t + LA);
        // (group 0 always exists: its MFMAs run unconditionally, so the compiler sees every
        // weight register of the stage consumed, its load complete, on every path)
        if (FULL || b == 0 || b < ngroups) {
#pragma unroll
          for (int a = 0; a < NF; ++a) acc[a][b] = mfma_step<WT>(W[a][f], cur, cur, acc[a][b]);
        }
      }
    }
  }

  // COH: the activation rows were written earlier in this launch (H), so they are read
  // with the device-coherent policy
  // WSTEP: bytes between consecutive 64-byte K steps of a weight fragment (kWStep for the
  // packed expert weights, 64 for the row-major router rows)
  // sbase, sstride (fp8 activations only): the rows' block scales, one byte per 128-wide
  // block, sstride bytes (a multiple of 4) per row; staged in LDS (lb.sl) before the K loop
  // sig: the completion counter of this workgroup's previous item, whose result stores may
  // still be in flight (null: none); it is incremented once every wave's stores have
  // completed, after this item's first loads are issued, so that their latency overlaps
  template <bool COH, int WSTEP>
  __device__ static void run(f4 (&acc)[NF][MG], const char *const (&wrow)[NF], const float *const (&sc)[NF],
                             const char *abase, size_t arow_bytes, const int *rows, const Lds3 &lb, int K,
                             int ngroups, const uint8_t *sbase = nullptr, int sstride = 0, int *sig = nullptr) {
    const int tid = otid(), lane = tid & 63, g = lane >> 4, j = lane & 15;
    const int wv = uni(tid >> 6);
    const int nch = K / KC;
#pragma unroll
    for (int a = 0; a < NF; ++a)
#pragma unroll
      for (int b = 0; b < MG; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

    if constexpr (WT == WQ8) {
      // the block scales of the tile's rows, row r at lb.sl + r * sstride: 4 bytes per lane per
      // load-to-LDS (lanes past the end repeat the last word into the buffer's padding); they
      // are the oldest loads of the wave, so the K loop's first wait covers them
      const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(sbase);
      const int dpr = sstride >> 2, nd = BMR * dpr;
      for (int w0 = wv * 64; w0 < nd; w0 += kWaves * 64) {
        const int w = min(w0 + lane, nd - 1), r = w / dpr;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (__attribute__((address_space(3))) void *)(lb.sl + 4 * w0), 4,
                                                 (uint32_t)(rows[r] * sstride + 4 * (w - r * dpr)), 0, 0,
                                                 COH ? kCpolSc1 : 0);
      }
    }
    // activation rows: one buffer resource at abase, a per-lane offset per load (the row's
    // 32-bit offset: every activation tensor is below 4 GB) and the chunk offset
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(abase);
    uint32_t aoff[NDMA];
#pragma unroll
    for (int s = 0; s < NDMA; ++s) {
      const int q = s * kWaves + wv;
      const int r = min(q * RPK + lane / NCOL, BMR - 1);  // (clamped for waves without DMA)
      const int col = (lane % NCOL) ^ (r & (NCOL - 1));
      aoff[s] = (uint32_t)((size_t)rows[r] * arow_bytes + col * 16);
    }
    // Prefetches past the last chunk still issue, so every pipeline stage has the same memory
    // operations: the wait counts stay constant and the compiler's register scoreboard stays
    // exact across the loop's back edge (a conditional prefetch makes it wait for everything).
    // Weight loads are buffer loads: one resource per fragment, based at lane 0's address of
    // that fragment (the fragments of a wave may lie in different matrices: gate and up), a
    // loop-invariant per-lane offset and the chunk offset in a scalar register, so no vector
    // register holds a per-stage address (the compiler cannot prove such a temporary free of
    // pending loads after the loop's back edge, and would wait for every outstanding load
    // before reusing it).  Lane 0 holds a fragment's lowest address (an expert fragment's
    // lanes are 16 bytes apart; a router fragment's lanes step through its 16 rows, clamped
    // to the last expert), so every offset is small and non-negative.
    __amdgpu_buffer_rsrc_t wrsrc[NF];
    uint32_t woff[NF];
#pragma unroll
    for (int a = 0; a < NF; ++a) {
      const char *base = reinterpret_cast<const char *>(uni64(reinterpret_cast<uint64_t>(wrow[a])));
      wrsrc[a] = make_rsrc(base);
      woff[a] = (uint32_t)(wrow[a] - base);
    }
    // (prefetches past the last chunk read the last chunk again: a clamped uniform offset keeps
    // the address arithmetic free of selects and temporaries, whose registers the compiler
    // could otherwise not prove free of pending loads, and would drain the pipeline for)
    auto dma = [&](int c, char *buf) {
      const uint32_t off = (uint32_t)(min(c, nch - 1) * RB);
      if (NKB >= kWaves || wv < NKB) {
#pragma unroll
        for (int s = 0; s < NDMA; ++s) dma16<COH>(arsrc, aoff[s], off, buf + (s * kWaves + wv) * 1024);
      }
    };
    // (expert weights are read once: nontemporal; the router's rows are read by every router
    // tile of the XCD, so they load with the default policy and stay in its L2)
    constexpr int wpol = WSTEP == kWStep ? kCpolNt : 0;
    auto ldw = [&](uint4(&W)[NF][FL], int c) {
      const int off = min(c, nch - 1) * (FL * WSTEP);
#pragma unroll
      for (int f = 0; f < FL; ++f)
#pragma unroll
        for (int a = 0; a < NF; ++a)
          W[a][f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc[a], woff[a], off + f * WSTEP, wpol));
    };
    // small tiles and the fp8-activation tiles compute every token group (rows past the
    // tile's end repeat its last row, valid data whose results are not stored); the other
    // large tiles skip absent groups, which also keeps the compiler from hoisting every LDS
    // read of the chunk at once
    auto compute = [&](const uint4(&W)[NF][FL], const char *A, int c) {
      asm volatile("" ::: "memory");  // the stage's prefetches are issued before its math
      chunk_mfma<(MG <= 2) || WT == WQ8>(acc, W, A, sc, c, ngroups, g, j, lb.sl, sstride);
    };
    // NBUF register/LDS stages, NBUF - 1 chunks in flight: each step waits only for its own
    // chunk (vmcnt counts this wave's outstanding operations, which complete in issue order,
    // so at most NBUF - 2 later chunks may remain), refills the stage freed by the previous
    // step (the barrier also tells every wave that this stage has been read by all of them),
    // then computes.  The loop body is unrolled over the stages, so every buffer index is a
    // constant and the weight stages stay in registers.
    uint4 W[NBUF][NF][FL];
#pragma unroll
    for (int st = 0; st < NBUF - 1; ++st) {
      dma(st, stage_buf(lb, st));
      ldw(W[st], st);
    }
    if (sig != nullptr) {
      // every operation older than the prologue's loads (the previous item's stores) has
      // completed in every wave once all waves pass the barrier (vmcnt counts in issue order)
      wait_vm<(NBUF - 1) * PER_CHUNK>();
      lds_barrier();
      if (otid() == 0) __hip_atomic_fetch_add(sig, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bool done = false;
    for (int c = 0;; c += NBUF) {
#pragma unroll
      for (int st = 0; st < NBUF; ++st) {
        wait_vm<(NBUF - 2) * PER_CHUNK>();
        lds_barrier();
        const int nx = (st + NBUF - 1) % NBUF;
        dma(c + st + NBUF - 1, stage_buf(lb, nx));
        ldw(W[nx], c + st + NBUF - 1);
        compute(W[st], stage_buf(lb, st), c + st);
        if (c + st + 1 >= nch) {
          done = true;
          break;
        }
      }
      if (done) break;
    }
    wait_vm0();  // the trailing prefetches land before the caller reuses the buffers
  }
};

// ---------------------------------------------------------------------------------
// shared memory
// ---------------------------------------------------------------------------------
// bytes of each activation staging buffer (separate LDS variables, see Lds3):
// the expert tile's chunk, or the router tile's on kernels whose router uses the tile core
template <int WT, int MG> struct ActBuf {
  using RC = Core<(WT == WF32 ? WF32 : WBF16), router_groups(MG)>;
  static constexpr int BYTES = (MG > 1 && RC::BUF > Core<WT, MG>::BUF) ? RC::BUF : Core<WT, MG>::BUF;
  // the third stage: the expert tiles' own where they have three stages, else only the router
  // tiles' (whose pipeline always has three)
  static constexpr int BYTES2 = Shape<WT, MG>::NBUF >= 3 ? BYTES : (MG > 1 && RC::BUF > 16 ? RC::BUF : 16);
};

template <int WT, int MG> struct Smem {
  union {
    struct {
      int16_t ids[kTopkTokens * kMaxK > kMaxChunkSlots ? kTopkTokens * kMaxK : kMaxChunkSlots];  // ids (-1: invalid)
      int hist[kMaxE];                         // per-expert slot counts of the chunk
      int tmp[kMaxE];                          // per-expert m-tile counts (plan)
      int scan0[kMaxE + 1];                    // offsets (plan)
      int scan1[kMaxE + 1];                    // m-tile offsets (plan); a chunk's base (scatter)
      int mto[kMaxE + 1];                      // m-tile offsets (scatter items)
      uint32_t mask[kMaxE][kMaxChunkTokens / 32];  // tokens of the chunk that chose expert e
    } r;
    f4 red[kWaves][64];
  } u;
  int rows[(MG > router_groups(MG) ? MG : router_groups(MG)) * 16];
  int bcast[4];
  uint32_t mark[2];  // trace: clock at the start and end of the tile loop of this item
};

// ---------------------------------------------------------------------------------
// workgroup-level sync helpers
// ---------------------------------------------------------------------------------
// Every thread: wait until this thread's device-coherent stores have completed, then (after
// the barrier) bump `counter` once.  Returns the counter's old value (thread 0 only).
__device__ __forceinline__ int wg_signal(int *counter) {
  wait_vm0();
  __syncthreads();
  int old = 0;
  if (otid() == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

template <class SM>
__device__ __forceinline__ bool wg_wait(const int *p, int target, int *err, SM &sm) {
  __syncthreads();
  if (otid() == 0) sm.bcast[1] = spin_geq(p, target, err) ? 1 : 0;
  __syncthreads();
  return uni(sm.bcast[1]) != 0;
}

// wg_wait for a workgroup that may hold a pending completion counter (pend, see gateup_item):
// when the wait is not already satisfied, the pending counter is incremented first (its
// item's stores waited for), since what this workgroup waits for may depend on it.
template <class SM>
__device__ __forceinline__ bool wg_wait_flush(const int *p, int target, int *err, SM &sm, int *&pend) {
  if (pend != nullptr) {
    __syncthreads();
    if (otid() == 0) sm.bcast[1] = ld_relaxed(p) >= target ? 1 : 0;
    __syncthreads();
    if (uni(sm.bcast[1])) return true;
    wg_signal(pend);
    pend = nullptr;
  }
  return wg_wait(p, target, err, sm);
}

// Publishes the plan: n_mt + 1 goes into every copy of the plan flag once this workgroup's
// plan (and scatter) stores have completed.  Most of the grid waits for the plan at the
// start of the layer; polls of one word would all queue at one memory channel and hold up
// every other access to it (the routing's own loads among them), so each workgroup polls
// a copy of its own.
__device__ __forceinline__ void plan_publish(const KParams &P, int nmt) {
  wait_vm0();
  __syncthreads();
  const int tid = otid();
  if (tid < kPlanCopies) st_coh(P.ctrl + plan_flag_word(tid), nmt + 1);
}

// Waits for the plan (this workgroup's copy of the flag); returns n_mt, or -1 on timeout.
template <class SM>
__device__ __forceinline__ int wg_wait_plan(const KParams &P, SM &sm) {
  __syncthreads();
  if (otid() == 0) {
    const int v = spin_value(P.ctrl + plan_flag_word((int)blockIdx.x % kPlanCopies), 1, P.ctrl + kSlotInts * C_ERR);
    sm.bcast[1] = v < 0 ? -1 : v - 1;
  }
  __syncthreads();
  return uni(sm.bcast[1]);
}

// ---------------------------------------------------------------------------------
// phase items
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void zero_item(const KParams &P, int i) {
  const int lo = i * kZeroPerItem;
  for (int q = otid(); q < kZeroPerItem; q += kThreads) {
    const int idx = lo + q;
    if (idx < P.gd_words) st_coh(P.gudone + idx, 0);
    else if (idx - P.gd_words < P.hist_words) st_coh(P.hist + (idx - P.gd_words), 0);
  }
}

// activation quantisation item (fp8 activations): tokens [16 q, 16 q + 16) of the hidden rows
// -> E4M3 codes in xq and, per 128-wide block, the exponent s (+ 127) of its power-of-two scale
// in xs (fp8_scale_exp of the block's largest magnitude; codes of v * 2^-s, nearest even).
// 16 lanes per block (8 values each), one token per 16 lanes (kQuantTokens = 16 lane groups of
// the workgroup); each lane issues the loads of kQuantBatch blocks before converting any (the
// rows are read once, so latency is what counts).  Lanes past the last block or token repeat
// it (same values, so the row max sees whole blocks) and store nothing.
constexpr int kQuantBatch = 28;
static_assert(kQuantTokens == 4 * kWaves, "one token per 16-lane group");
// max over the 16 lanes of a DPP row, in every lane: quad swaps (xor 1, xor 2), then the
// mirrored half row and row (vector ALU permutes instead of four LDS-routed shuffles)
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float row_max16(float v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  return dpp_max<0x140>(v);  // row_mirror
}
__device__ __forceinline__ void quant_item(const KParams &P, int q) {
  const int tid = otid(), lane = tid & 63, l16 = lane & 15;
  // lane group s (16 lanes) quantises token t0 + s, kQuantBatch blocks per pass in K order
  // (no index division); each lane holds 8 consecutive values of a 128-wide block
  const int slot = (tid >> 6) * 4 + (lane >> 4);
  const int nblk = P.d >> 7, t0 = q * kQuantTokens, nt = min(kQuantTokens, P.T - t0);
  const bool live = slot < nt;
  const size_t t = (size_t)(t0 + min(slot, nt - 1));  // (rows past the end repeat the last)
  const uint16_t *xr = reinterpret_cast<const uint16_t *>(P.x) + t * P.d + 8 * l16;
  uint8_t *qr = P.xq + t * P.d + 8 * l16;
  for (int kb0 = 0; kb0 < nblk; kb0 += kQuantBatch) {
    uint4 v[kQuantBatch];
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) v[u] = ld_glob16(xr + min(kb0 + u, nblk - 1) * 128);
#pragma unroll
    for (int u = 0; u < kQuantBatch; ++u) {
      const int kb = kb0 + u;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
      float mx = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
      mx = row_max16(mx);
      const int se = fp8_scale_exp(mx);
      if (live && kb < nblk) {
        const uint64_t codes = (uint64_t)fp8x4(f[0], f[1], f[2], f[3], se) |
                               ((uint64_t)fp8x4(f[4], f[5], f[6], f[7], se) << 32);
        st_coh64(qr + kb * 128, codes);
        if (l16 == 0) st_coh8(P.xs + t * P.xs_stride + kb, (uint32_t)(se + 127));
      }
    }
  }
}

// router logits, decode-sized tiles: 16 tokens x 16 experts over part ks of S = rt_split
// equal parts of K; wave w sums the w-th quarter of that part, then the four partial sums
// are added in wave order.  With S == 1 the item adds the bias and writes the logits; else
// it writes its partial sums to lpart[ks], and the top-k items add the S parts in order.
// Latency matters here (the rest of the layer waits for the routing), so each wave issues
// all of its loads of a 16-step chunk (and the bias) before the first MFMA: one memory
// round trip per chunk.  Steps past the end read the last step again and multiply zero
// activations.
template <int WT, class SM>
__device__ __forceinline__ void logits_item_split(const KParams &P, int i, SM &sm) {
  constexpr int RT = (WT == WF32) ? WF32 : WBF16;  // the router runs in the activation dtype
  constexpr int KU = Ty<RT>::KU, ASZ = Ty<RT>::ASZ;
  constexpr int CH = 16;  // K steps per chunk
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int S = P.rt_split, ls = S == 8 ? 3 : S == 4 ? 2 : S == 2 ? 1 : 0;  // (S: 1, 2, 4 or 8)
  const int ks = i & (S - 1), tile = i >> ls;
  const int lt = tile / P.n_le, le = tile % P.n_le;
  const int t0 = lt * 16, e0 = le * 16;
  const int kq = P.d >> (2 + ls), kbeg = ks * (P.d >> ls) + wv * kq;
  const int er = min(e0 + j, P.E - 1), tr = min(t0 + j, P.T - 1);
  const char *wp = reinterpret_cast<const char *>(P.wr) + ((size_t)er * P.d + kbeg) * ASZ + g * 16;
  const char *xp = reinterpret_cast<const char *>(P.x) + ((size_t)tr * P.d + kbeg) * ASZ + g * 16;
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (P.bias && S == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[r] = P.bias[min(e0 + 4 * g + r, P.E - 1)];
  }
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  const int nsteps = kq / KU;
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  int s0 = 0;
  // full chunks: one base address each, the steps at immediate offsets (short code, which
  // matters here: the item runs once per layer, so its instructions are fetched cold)
  for (; s0 + CH <= nsteps; s0 += CH) {
    uint4 w[CH], a[CH];
    const char *wc = wp + (size_t)s0 * 64, *xc = xp + (size_t)s0 * 64;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      w[u] = ld_glob16(wc + u * 64);
      a[u] = ld_glob16(xc + u * 64);
    }
    asm volatile("" ::: "memory");  // every load of the chunk is in flight before the first MFMA
#pragma unroll
    for (int u = 0; u < CH; ++u) acc = mfma_step<RT>(w[u], a[u], a[u], acc);
  }
  if (s0 < nsteps) {  // last, partial chunk
    uint4 w[CH], a[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const size_t off = (size_t)min(s0 + u, nsteps - 1) * 64;
      w[u] = ld_glob16(wp + off);
      a[u] = ld_glob16(xp + off);
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const uint4 av = s0 + u < nsteps ? a[u] : z4;
      acc = mfma_step<RT>(w[u], av, av, acc);
    }
  }
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  sm.u.red[wv][lane] = acc;
  __syncthreads();
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  if (wv == 0) {
    const f4 sum = ((sm.u.red[0][lane] + sm.u.red[1][lane]) + sm.u.red[2][lane]) + sm.u.red[3][lane];
    const int t = t0 + j;
    if (t < P.T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 4 * g + r;
        if (e >= P.E) continue;
        if (S == 1) st_coh(P.logits + (size_t)t * P.E + e, sum[r] + bias[r]);
        else st_coh(P.lpart + ((size_t)ks * P.T + t) * P.E + e, sum[r]);
      }
    }
  }
}

// router logits, wide tiles: 16 tokens x 128 experts on the expert tile core (router rows
// are the weight operand, token rows the activation operand)
template <int WT, int MG, class SM>
__device__ __forceinline__ void logits_item_tile(const KParams &P, int i, SM &sm, const Lds3 &lb) {
  constexpr int RT = (WT == WF32) ? WF32 : WBF16;
  // 16 * RMG tokens x 64 * NF experts per tile (W_r is read once per tile's tokens), over
  // part ks of the S = rt_split parts of K (enough items to spread over the GPU); S > 1
  // writes partial sums that the top-k items add in part order, then the bias
  constexpr int RMG = router_groups(MG);
  using C = Core<RT, RMG>;
  constexpr int NF = C::NF;
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int S = P.rt_split, ls = S == 8 ? 3 : S == 4 ? 2 : S == 2 ? 1 : 0;  // (S: 1, 2, 4 or 8)
  const int ks = i & (S - 1), tile = i >> ls;
  const int lt = tile / P.n_le, le = tile % P.n_le;
  const int kpart = P.d >> ls, kbeg = ks * kpart;
  const int t0 = lt * C::BMR, e0 = le * (64 * NF) + wv * 16 * NF;
  const int m = min(C::BMR, P.T - t0);
  for (int r = tid; r < C::BMR; r += kThreads) sm.rows[r] = t0 + min(r, m - 1);
  __syncthreads();
  const size_t asz = Ty<RT>::ASZ;
  const char *wrow[NF];
  const float *sc[NF];
#pragma unroll
  for (int a = 0; a < NF; ++a) {
    const int er = min(e0 + 16 * a + j, P.E - 1);
    wrow[a] = reinterpret_cast<const char *>(P.wr) + ((size_t)er * P.d + kbeg) * asz + g * 16;
    sc[a] = nullptr;
  }
  f4 acc[NF][RMG];
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  C::template run<false, 64>(acc, wrow, sc, reinterpret_cast<const char *>(P.x) + (size_t)kbeg * asz,
                             (size_t)P.d * asz, sm.rows, lb, kpart, (m + 15) >> 4);
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  // The sums leave through LDS, so that a store covers whole runs of a token's row: per
  // 16-token group, the wave's NF fragments (16 tokens x its EPW experts) go to its own slab
  // of the routing scratch (unused by this item; rows padded by 4 floats against bank
  // conflicts), and each lane then stores 4 consecutive experts of one token, LPR lanes
  // covering the wave's contiguous 4 * EPW bytes of that token's row.  (A wave reads back
  // only what its own lanes wrote, and its LDS operations complete in order.)
  constexpr int EPW = 16 * NF, LPR = EPW / 4, RPI = 64 / LPR, SROW = EPW + 4;
  static_assert(sizeof(sm.u) >= kWaves * 16 * SROW * sizeof(float), "router tile slab");
  float *slab = reinterpret_cast<float *>(&sm.u) + wv * 16 * SROW;
  float bv[4] = {0.f, 0.f, 0.f, 0.f};
  const int col = (lane % LPR) * 4, e = e0 + col;
  if (P.bias && S == 1) {
#pragma unroll
    for (int z = 0; z < 4; ++z) bv[z] = e + z < P.E ? P.bias[e + z] : 0.f;
  }
  float *const dst = S == 1 ? P.logits : P.lpart + (size_t)ks * P.T * P.E;
  // four consecutive logits of a token as one 16-byte device-coherent store (a buffer
  // resource at the tile's first token row: the tile's rows span at most 64 rows of E floats)
  // when all four are in range and 16-byte aligned, else one by one
  const bool vec = e + 3 < P.E && (P.E & 3) == 0;
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(dst + (size_t)t0 * P.E);
#pragma unroll
  for (int b = 0; b < RMG; ++b) {
    if (b * 16 >= m) break;
#pragma unroll
    for (int a = 0; a < NF; ++a) *reinterpret_cast<f4 *>(slab + j * SROW + 16 * a + 4 * g) = acc[a][b];
#pragma unroll
    for (int q = 0; q < 16 / RPI; ++q) {
      const int row = q * RPI + lane / LPR;
      const f4 v = *reinterpret_cast<const f4 *>(slab + row * SROW + col);
      if (b * 16 + row >= m || e >= P.E) continue;
      float *p = dst + (size_t)(t0 + b * 16 + row) * P.E + e;
      if (vec) {
        const u32x4 q = {__float_as_uint(v[0] + bv[0]), __float_as_uint(v[1] + bv[1]), __float_as_uint(v[2] + bv[2]),
                         __float_as_uint(v[3] + bv[3])};
        __builtin_amdgcn_raw_buffer_store_b128(q, lrs, (uint32_t)(((b * 16 + row) * P.E + e) * 4), 0, kCpolSc1);
      } else {
#pragma unroll
        for (int z = 0; z < 4; ++z)
          if (e + z < P.E) st_coh(p + z, v[z] + bv[z]);
      }
    }
  }
}

// wave-level exclusive scan of in[0..N) -> out[0..N] (out[N] = total); one wave runs it
__device__ __forceinline__ void wave_excl_scan(const int *in, int *out, int N, int lane) {
  const int per = (N + 63) / 64;
  const int lo = min(lane * per, N), hi = min(lo + per, N);
  int s = 0;
  for (int q = lo; q < hi; ++q) s += in[q];
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  int run = incl - s;
  for (int q = lo; q < hi; ++q) {
    out[q] = run;
    run += in[q];
  }
  if (lane == 63) out[N] = incl;
}

// wave-wide unsigned max of N independent 32-bit values (each returned in every lane):
// row-shift and row-broadcast DPP steps (VALU data movement, no LDS round trips), the N
// reductions interleaved step by step so that their latencies overlap; out-of-row lanes
// read 0 (the identity of unsigned max), which lets each step be a single DPP max
template <int N>
__device__ __forceinline__ void wave_max_u32(uint32_t (&v)[N]) {
#define MOE_DPP_MAX(CTRL, ROWM, BANKM)                                                      \
  _Pragma("unroll") for (int i = 0; i < N; ++i) {                                          \
    const uint32_t o = __builtin_amdgcn_update_dpp(0u, v[i], CTRL, ROWM, BANKM, true);    \
    v[i] = o > v[i] ? o : v[i];                                                            \
  }
  MOE_DPP_MAX(0x111, 0xf, 0xf)  // row_shr:1
  MOE_DPP_MAX(0x112, 0xf, 0xf)  // row_shr:2
  MOE_DPP_MAX(0x113, 0xf, 0xf)  // row_shr:3
  MOE_DPP_MAX(0x114, 0xf, 0xe)  // row_shr:4
  MOE_DPP_MAX(0x118, 0xf, 0xc)  // row_shr:8
  MOE_DPP_MAX(0x142, 0xa, 0xf)  // row_bcast:15
  MOE_DPP_MAX(0x143, 0xc, 0xf)  // row_bcast:31
#undef MOE_DPP_MAX
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_readlane(v[i], 63);
}

// The plan: counts -> offsets (exclusive scan), m-tile counts -> m-tile offsets and the
// m-tile descriptor table.  One workgroup.  from_lds: the single chunk's histogram is in
// sm.u.r.hist (no global round trip); else the counts are the sums of the chunk histograms
// (which the scatter items read too, for their own chunk's base).
template <class SM>
__device__ __forceinline__ void plan_wg(const KParams &P, SM &sm, bool from_lds) {
  const int tid = otid(), E = P.E, nkc = P.n_kc;
  int *cnt = sm.u.r.hist;
  int *mtc = sm.u.r.tmp;
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
    if (from_lds) {
      run = cnt[e];
    } else {
      for (int c0 = 0; c0 < nkc; c0 += 32) {
        int h[32];
#pragma unroll
        for (int q = 0; q < 32; ++q) h[q] = (c0 + q < nkc) ? ld_coh(P.hist + (size_t)(c0 + q) * E + e) : 0;
#pragma unroll
        for (int q = 0; q < 32; ++q) run += h[q];
      }
    }
    cnt[e] = run;
    mtc[e] = (run + P.bm - 1) / P.bm;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  int *soff = sm.u.r.scan0;
  int *smt = sm.u.r.scan1;
  if (wave == 0) wave_excl_scan(cnt, soff, E, lane);
  if (wave == 1) wave_excl_scan(mtc, smt, E, lane);
  __syncthreads();
  for (int e = tid; e <= E; e += kThreads) {
    st_coh(P.offsets + e, soff[e]);
    st_coh(P.mtoff + e, smt[e]);
  }
  for (int e = tid; e < E; e += kThreads) {
    st_coh(P.counts + e, cnt[e]);
    const int base = smt[e], off = soff[e], c = cnt[e];
    for (int mt = 0; mt < mtc[e]; ++mt) st_coh_int4(P.desc + base + mt, make_int4(e, off + mt * P.bm, min(P.bm, c - mt * P.bm), 0));
  }
}

// an expert id as kept in LDS: out-of-range ids (caller input) become -1 and are reported
__device__ __forceinline__ int16_t checked_id(int e, int E) { return (int16_t)((e >= 0 && e < E) ? e : -1); }

// chunk histogram and per-expert token bitmasks from the chunk's ids in sm.u.r.ids
template <class SM>
__device__ __forceinline__ void chunk_masks(const KParams &P, int ntok, SM &sm) {
  const int tid = otid(), k = P.k, E = P.E;
  for (int e = tid; e < E; e += kThreads) {
    sm.u.r.hist[e] = 0;
#pragma unroll
    for (int w = 0; w < kMaxChunkTokens / 32; ++w) sm.u.r.mask[e][w] = 0u;
  }
  __syncthreads();
  for (int q = tid; q < ntok * k; q += kThreads) {
    const int e = sm.u.r.ids[q];
    bool bad = e < 0 || e >= E;
    if (!bad) {
      // a token holds an expert at most once: a bit already set is a repeated id (caller
      // input), counted once and reported
      const int tt = q / k;
      const uint32_t bit = 1u << (tt & 31);
      if (atomicOr(&sm.u.r.mask[e][tt >> 5], bit) & bit) bad = true;
      else atomicAdd(&sm.u.r.hist[e], 1);
    }
    if (bad) __hip_atomic_store(P.ctrl + kSlotInts * C_ERR, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// stable scatter of a chunk: slot (t, j) with expert e goes to
//   offsets[e] + base[e] + #(earlier tokens of the chunk that chose e)
// (a token chooses an expert at most once, so the rank is a popcount of the mask).
// mto: per-expert m-tile offsets; the slot's m-tile (row r of expert e's rows is in m-tile
// mto[e] + r / bm) goes to slotmt, and with 16-row m-tiles the slot's token also goes to the
// m-tile token table
// TOK_ONLY: only the m-tile token table (16-row m-tiles); !WITH_TOK: everything else.
template <bool TOK_ONLY = false, bool WITH_TOK = true, class SM>
__device__ __forceinline__ void chunk_scatter(const KParams &P, int c, int ntok, const int *offs, const int *base,
                                              const int *mto, SM &sm) {
  const int tid = otid(), k = P.k, E = P.E, t0 = c * P.tk;
  for (int q = tid; q < ntok * k; q += kThreads) {
    const int e = sm.u.r.ids[q];
    if (e < 0 || e >= E) continue;
    const int tt = q / k;
    int rank = 0;
#pragma unroll
    for (int w = 0; w < kMaxChunkTokens / 32; ++w) {
      const uint32_t mw = sm.u.r.mask[e][w];
      if (w < (tt >> 5)) rank += __popc(mw);
      else if (w == (tt >> 5)) rank += __popc(mw & ((1u << (tt & 31)) - 1u));
    }
    const int r = (base ? base[e] : 0) + rank, p = offs[e] + r;
    const int slot = t0 * k + q;
    const int gm = mto[e] + r / P.bm;
    if (TOK_ONLY) {
      st_coh(P.mtok + gm * 16 + (r & 15), t0 + tt);
      continue;
    }
    st_coh(P.perm + p, slot);
    st_coh(P.inv_perm + slot, p);
    if (P.phases & PH_FFN) {
      st_coh(P.slotmt + slot, gm);
      if (WITH_TOK && P.bm == 16) st_coh(P.mtok + gm * 16 + (r & 15), t0 + tt);
    }
  }
}

// gate weights of TPW selected tokens: the softmax of the kept logits, summed in slot order.
// k <= 64: slot j's logit and id are in lane j; k > 64: the ids are in LDS and the logits
// are read again from memory (the same values, -0.0 read as +0.0).
template <int TPW>
__device__ __forceinline__ void topk_weights(const KParams &P, const int (&t)[TPW], const bool (&live)[TPW],
                                             const float (&lj)[TPW], const int (&ej)[TPW],
                                             int16_t *const (&ids_lds)[TPW]) {
  const int lane = otid() & 63, k = P.k, E = P.E;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    if (!live[u]) continue;
    if (k <= 64) {
      const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lj[u]), 0));
      const float z = lane < k ? expf(lj[u] - l0) : 0.f;
      float ssum = 0.f;
      for (int jj = 0; jj < k; ++jj) ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), jj));
      if (lane < k) {
        st_coh(P.wts + (size_t)t[u] * k + lane, z / ssum);
        st_coh(P.ids + (size_t)t[u] * k + lane, ej[u]);
      }
    } else {
      if (P.rt_split > 1) wait_vm0();  // this wave's own logits stores (split router)
      if (lane != 0) continue;
      const float *Lr = P.logits + (size_t)t[u] * E;
      const float l0 = ld_coh(Lr + ids_lds[u][0]) + 0.0f;
      float ssum = 0.f;
      for (int jj = 0; jj < k; ++jj) ssum += expf((ld_coh(Lr + ids_lds[u][jj]) + 0.0f) - l0);
      for (int jj = 0; jj < k; ++jj) {
        const int e = ids_lds[u][jj];
        st_coh(P.wts + (size_t)t[u] * k + jj, expf((ld_coh(Lr + e) + 0.0f) - l0) / ssum);
        st_coh(P.ids + (size_t)t[u] * k + jj, e);
      }
    }
  }
}

// top-k of TPW tokens on one wave, in lockstep (their reductions are independent, so they
// overlap).  Lane l holds the keys of experts l, l + 64, ... (NQ of them): the ordered
// 32-bit image of the logit, 0 for absent or already taken experts.  Each round takes the
// largest key (wave max), then the lowest expert id holding it (wave min), which is the
// (logit descending, id ascending) order.  Slot j's id and logit stay in lane j (k <= 64);
// the gate weights are the softmax of the kept logits, summed in slot order.
template <int NQ, int TPW>
__device__ __forceinline__ void topk_group(const KParams &P, const int (&t)[TPW], const bool (&live)[TPW],
                                           uint32_t (&key)[TPW][NQ], int16_t *const (&ids_lds)[TPW]) {
  const int lane = otid() & 63, k = P.k, E = P.E;
  float lj[TPW];
  int ej[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    lj[u] = 0.f;
    ej[u] = 0;
  }
  for (int jj = 0; jj < k; ++jj) {
    uint32_t m[TPW], c[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      uint32_t b = key[u][0];
#pragma unroll
      for (int q = 1; q < NQ; ++q) b = key[u][q] > b ? key[u][q] : b;
      m[u] = b;
    }
    wave_max_u32<TPW>(m);
    // the lowest id holding the maximum: the max of the complemented ids (0 = no match)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      uint32_t x = 0u;
#pragma unroll
      for (int q = NQ - 1; q >= 0; --q)
        if (key[u][q] == m[u]) x = ~(uint32_t)(q * 64 + lane);  // this lane's lowest matching id
      c[u] = x;
    }
    wave_max_u32<TPW>(c);
#pragma unroll
    for (int u = 0; u < TPW; ++u) c[u] = ~c[u];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if ((uint32_t)(q * 64 + lane) == c[u]) key[u][q] = 0u;
      if (lane == (jj & 63)) {
        lj[u] = key_value(m[u]);
        ej[u] = (int)c[u];
      }
      if (lane == 0 && live[u]) ids_lds[u][jj] = (int16_t)c[u];
    }
  }
  topk_weights<TPW>(P, t, live, lj, ej, ids_lds);
}

// Selection of the same order for E <= 256 (4 keys per lane), with about half the work per
// round.  Each lane first sorts its 4 keys, largest first; the adjacent compare-exchanges
// swap only on a strictly larger key, so equal keys keep their increasing expert ids.  A
// round then needs one wave max over the lanes' heads: the lanes whose head equals it are
// a ballot, and when only one lane holds the maximum (the usual case) its head is the
// winner.  Several tied lanes take the lowest id among their heads (wave max of the
// complemented ids).  The winning lane drops its head.  Slot j's id and logit land in
// lane j (k <= 64); for k > 64 lane 0 also writes the ids to LDS.
// V4: lane l holds experts 4 l .. 4 l + 3 (key q is expert 4 l + q), else experts l, l + 64,
// l + 128, l + 192 (key q is expert 64 q + l); either way a lane's keys start in increasing
// expert order, which the stable sort keeps for equal keys
template <int TPW, bool V4>
__device__ __forceinline__ void topk_group4(const KParams &P, const int (&t)[TPW], const bool (&live)[TPW],
                                            uint32_t (&key)[TPW][4], int16_t *const (&ids_lds)[TPW]) {
  const int lane = otid() & 63, k = P.k;
  int qq[TPW][4];
  float lj[TPW];
  int ej[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    lj[u] = 0.f;
    ej[u] = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) qq[u][q] = q;
  }
  auto cx = [&](int u, int a, int b) {
    const bool sw = key[u][b] > key[u][a];
    const uint32_t ka = key[u][a], kb = key[u][b];
    const int qa = qq[u][a], qb = qq[u][b];
    key[u][a] = sw ? kb : ka;
    key[u][b] = sw ? ka : kb;
    qq[u][a] = sw ? qb : qa;
    qq[u][b] = sw ? qa : qb;
  };
#pragma unroll
  for (int u = 0; u < TPW; ++u) {  // odd-even transposition sort: 4 rounds for 4 keys
    cx(u, 0, 1);
    cx(u, 2, 3);
    cx(u, 1, 2);
    cx(u, 0, 1);
    cx(u, 2, 3);
    cx(u, 1, 2);
  }
  for (int jj = 0; jj < k; ++jj) {
    uint32_t m[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) m[u] = key[u][0];
    wave_max_u32<TPW>(m);
    uint64_t tie[TPW];
    bool many = false;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      tie[u] = __builtin_amdgcn_ballot_w64(key[u][0] == m[u]);
      many |= __builtin_popcountll(tie[u]) > 1;
    }
    int win[TPW];
    if (many) {
      uint32_t c[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        c[u] = key[u][0] == m[u] ? ~(uint32_t)(V4 ? lane * 4 + qq[u][0] : qq[u][0] * 64 + lane) : 0u;
      wave_max_u32<TPW>(c);
#pragma unroll
      for (int u = 0; u < TPW; ++u) win[u] = (int)~c[u];
    } else {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int wl = (int)__builtin_ctzll(tie[u]);
        const int wq = __builtin_amdgcn_readlane(qq[u][0], wl);
        win[u] = V4 ? wl * 4 + wq : wq * 64 + wl;
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const bool pop = lane == (V4 ? win[u] >> 2 : win[u] & 63);
      key[u][0] = pop ? key[u][1] : key[u][0];
      key[u][1] = pop ? key[u][2] : key[u][1];
      key[u][2] = pop ? key[u][3] : key[u][2];
      key[u][3] = pop ? 0u : key[u][3];
      qq[u][0] = pop ? qq[u][1] : qq[u][0];
      qq[u][1] = pop ? qq[u][2] : qq[u][1];
      qq[u][2] = pop ? qq[u][3] : qq[u][2];
      if (lane == (jj & 63)) {
        lj[u] = key_value(m[u]);
        ej[u] = win[u];
      }
    }
    if (k > 64) {
#pragma unroll
      for (int u = 0; u < TPW; ++u)
        if (lane == 0 && live[u]) ids_lds[u][jj] = (int16_t)win[u];
    }
  }
  if (k <= 64) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
      if (live[u] && lane < k) ids_lds[u][lane] = (int16_t)ej[u];
  }
  topk_weights<TPW>(P, t, live, lj, ej, ids_lds);
}

// top-k + softmax for the ntok <= 4 * TPW tokens of an item.  For E <= 256 a wave handles
// its TPW tokens together, with all of their logits loaded before the first selection.  The
// loads are unconditional (clamped index, masked after): a load under a lane condition is
// waited for inside its branch, which would serialise the loads.
// SMAX: the most parts the router's K can be split into in this kernel
// V4 (E a multiple of 4): a lane holds 4 consecutive experts' logits, read as one 16-byte
// load per token and K part (else 4 loads 64 experts apart)
template <int TPW, int SMAX, bool V4, class SM>
__device__ __forceinline__ void topk_tokens(const KParams &P, int t0, int ntok, SM &sm) {
  const int tid = otid(), wave = tid >> 6, lane = tid & 63, k = P.k, E = P.E;
  auto eid = [&](int q) { return V4 ? lane * 4 + q : q * 64 + lane; };
  // 16-byte device-coherent load of 4 logits of a row (row: wave-uniform); lanes past E read
  // the row's last 4 (their keys are dropped)
  auto ld4 = [&](const float *row) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(uni64(reinterpret_cast<uint64_t>(row))));
    return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(min(lane * 4, E - 4) * 4), 0, kCpolSc1));
  };
  if (E <= 256) {
    float v[TPW][4];
    int t[TPW];
    bool live[TPW];
    int16_t *ids[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = wave + u * kWaves;
      live[u] = tt < ntok;
      t[u] = t0 + min(tt, ntok - 1);
      ids[u] = sm.u.r.ids + tt * k;
    }
    // split router (rt_split > 1): lpart holds the K parts of the logits, added here in part
    // order, then the bias; the finished logits are written out (the routing's logits
    // output; the k > 64 path reads them back)
    const int S = P.rt_split;
    const float *L0 = S == 1 ? P.logits : P.lpart;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const float *Lr = L0 + (size_t)t[u] * E;
      if constexpr (V4) {
        const f4 r = ld4(Lr);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u][q] = r[q];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u][q] = ld_coh(Lr + min(eid(q), E - 1));
      }
    }
    asm volatile("" ::: "memory");  // all of the wave's loads are in flight before any is used
    if (S > 1) {
      // parts 1..S-1 loaded together (clamped part index; unused copies are not added)
      float pp[TPW][4][SMAX - 1];
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int x = 0; x < SMAX - 1; ++x) {
          const float *Lp = P.lpart + ((size_t)min(x + 1, S - 1) * P.T + t[u]) * E;
          if constexpr (V4) {
            const f4 r = ld4(Lp);
#pragma unroll
            for (int q = 0; q < 4; ++q) pp[u][q][x] = r[q];
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) pp[u][q][x] = ld_coh(Lp + min(eid(q), E - 1));
          }
        }
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int x = 0; x < SMAX - 1; ++x)
            if (x + 1 < S) v[u][q] += pp[u][q][x];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float bq = P.bias ? P.bias[min(eid(q), E - 1)] : 0.f;
#pragma unroll
        for (int u = 0; u < TPW; ++u) v[u][q] += bq;
      }
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        if (!live[u]) continue;
        float *Lo = P.logits + (size_t)t[u] * E;
        if constexpr (V4) {
          if (lane * 4 < E) {
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(reinterpret_cast<const char *>(uni64(reinterpret_cast<uint64_t>(Lo))));
            const u32x4 o = {__float_as_uint(v[u][0]), __float_as_uint(v[u][1]), __float_as_uint(v[u][2]),
                             __float_as_uint(v[u][3])};
            __builtin_amdgcn_raw_buffer_store_b128(o, rs, (uint32_t)(lane * 16), 0, kCpolSc1);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (eid(q) < E) st_coh(Lo + eid(q), v[u][q]);
        }
      }
    }
    uint32_t key[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) key[u][q] = (eid(q) < E) ? ordered_key(v[u][q]) : 0u;
    topk_group4<TPW, V4>(P, t, live, key, ids);
  } else {
    for (int tt = wave; tt < ntok; tt += kWaves) {
      const int t[1] = {t0 + tt};
      const bool live[1] = {true};
      int16_t *const ids[1] = {sm.u.r.ids + tt * k};
      const float *Lr = P.logits + (size_t)t[0] * E;
      float v[kMaxE / 64];
      if (P.rt_split == 1) {
#pragma unroll
        for (int q = 0; q < kMaxE / 64; ++q) v[q] = ld_coh(Lr + min(q * 64 + lane, E - 1));
      } else {
#pragma unroll
        for (int q = 0; q < kMaxE / 64; ++q) {
          const int e = min(q * 64 + lane, E - 1);
          float x = ld_coh(P.lpart + (size_t)t[0] * E + e);
          for (int ks = 1; ks < P.rt_split; ++ks) x += ld_coh(P.lpart + ((size_t)ks * P.T + t[0]) * E + e);
          x += P.bias ? P.bias[e] : 0.f;
          v[q] = x;
          if (q * 64 + lane < E) st_coh(P.logits + (size_t)t[0] * E + e, x);
        }
      }
      uint32_t key[1][kMaxE / 64];
#pragma unroll
      for (int q = 0; q < kMaxE / 64; ++q) key[0][q] = (q * 64 + lane < E) ? ordered_key(v[q]) : 0u;
      topk_group<kMaxE / 64, 1>(P, t, live, key, ids);
    }
  }
}

// topk_tokens with its part loads sized for the router's actual K split (each load in flight
// holds a slot of the wave's limited count of outstanding memory operations)
template <int TPW, int SMAX, class SM>
__device__ __forceinline__ void topk_tokens_parts(const KParams &P, int t0, int ntok, SM &sm) {
  if ((P.E & 3) != 0) topk_tokens<TPW, SMAX, false>(P, t0, ntok, sm);  // (rare: E not a multiple of 4)
  else if (P.rt_split <= 2 || SMAX <= 2) topk_tokens<TPW, (SMAX < 2 ? SMAX : 2), true>(P, t0, ntok, sm);
  else if (P.rt_split <= 4 || SMAX <= 4) topk_tokens<TPW, (SMAX < 4 ? SMAX : 4), true>(P, t0, ntok, sm);
  else topk_tokens<TPW, SMAX, true>(P, t0, ntok, sm);
}

// K item c: top-k of kt_tok tokens.  When all tokens form one scatter chunk (n_kc == 1),
// the last K item to finish (or the only one) builds the plan and scatters every token;
// otherwise an item adds its per-expert counts to its chunk's histogram (integer atomics:
// order-independent), the last K item plans, and scatter items follow.
template <int SMAX, class SM>
__device__ __forceinline__ void topk_item(const KParams &P, int c, SM &sm) {
  const int tid = otid(), k = P.k, E = P.E;
  const int t0 = c * P.kt_tok, ntok = min(P.kt_tok, P.T - t0);
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  if (P.phases & PH_IDS_GIVEN) {
    for (int q = tid; q < ntok * k; q += kThreads) sm.u.r.ids[q] = checked_id(P.ids[(size_t)t0 * k + q], E);  // caller's input
  } else if (P.kt_tok == kTopkTokensSmall) {
    topk_tokens_parts<kTopkTokensSmall / kWaves, SMAX>(P, t0, ntok, sm);
  } else {
    topk_tokens_parts<kTopkTokens / kWaves, SMAX>(P, t0, ntok, sm);
  }
  __syncthreads();
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  if (!(P.phases & PH_PERMUTE)) {
    wg_signal(P.ctrl + kSlotInts * C_KDONE);
    return;
  }
  if (P.n_kc <= 1) {
    int nt = ntok;
    if (P.n_kt > 1) {
      // every item's ids and weights are stored once the counter shows all n_kt items
      const int old = wg_signal(P.ctrl + kSlotInts * C_KDONE);
      if (tid == 0) sm.bcast[2] = (old == P.n_kt - 1) ? 1 : 0;
      __syncthreads();
      if (!uni(sm.bcast[2])) return;
      nt = P.T;
      for (int q = tid; q < nt * k; q += kThreads) sm.u.r.ids[q] = checked_id(ld_coh(P.ids + q), E);
      __syncthreads();
    }
    chunk_masks(P, nt, sm);
    plan_wg(P, sm, true);
    __syncthreads();
    if ((P.phases & PH_FFN) && P.bm == 16) {
      // the gate/up units need only the plan and the m-tile token table: publish those
      // first, then finish the scatter (perm, inv_perm, slot m-tiles: for the combine)
      chunk_scatter<true>(P, 0, nt, sm.u.r.scan0, nullptr, sm.u.r.scan1, sm);
      plan_publish(P, sm.u.r.scan1[E]);
      chunk_scatter<false, false>(P, 0, nt, sm.u.r.scan0, nullptr, sm.u.r.scan1, sm);
    } else {
      chunk_scatter(P, 0, nt, sm.u.r.scan0, nullptr, sm.u.r.scan1, sm);
      plan_publish(P, sm.u.r.scan1[E]);
    }
    wg_signal(P.ctrl + kSlotInts * C_SDONE);  // (the combine waits for the whole scatter)
    return;
  }
  chunk_masks(P, ntok, sm);
  if (P.tk % kTopkTokens == 0) {  // the item lies in one chunk: add its histogram
    const int chunk = t0 / P.tk;
    for (int e = tid; e < E; e += kThreads) {
      const int h = sm.u.r.hist[e];
      if (h) __hip_atomic_fetch_add(P.hist + (size_t)chunk * E + e, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {  // large k: small chunks, one increment per slot
    for (int q = tid; q < ntok * k; q += kThreads) {
      const int e = sm.u.r.ids[q];
      if (e >= 0 && e < E)
        __hip_atomic_fetch_add(P.hist + (size_t)((t0 + q / k) / P.tk) * E + e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const int old = wg_signal(P.ctrl + kSlotInts * C_KDONE);
  if (tid == 0) sm.bcast[2] = (old == P.n_kt - 1) ? 1 : 0;
  __syncthreads();
  if (uni(sm.bcast[2])) {
    plan_wg(P, sm, false);
    plan_publish(P, sm.u.r.scan1[E]);
  }
}

// scatter of chunk c (several chunks): rebuild the chunk's masks from its ids
template <class SM>
__device__ __forceinline__ void scatter_item(const KParams &P, int c, SM &sm) {
  const int tid = otid(), k = P.k, E = P.E;
  const int t0 = c * P.tk, ntok = min(P.tk, P.T - t0);
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  for (int q = tid; q < ntok * k; q += kThreads) sm.u.r.ids[q] = checked_id(ld_coh(P.ids + (size_t)t0 * k + q), E);
  __syncthreads();
  chunk_masks(P, ntok, sm);
  // from the chunk histograms (complete once every top-k item is done), the same numbers the
  // plan holds: per expert, the rows of earlier chunks (this chunk's base), the total (whose
  // exclusive scan is the expert offsets) and its m-tile count (scan: m-tile offsets)
  const int nkc = P.n_kc;
  for (int e = tid; e < E; e += kThreads) {
    int base = 0, total = 0;
    for (int c0 = 0; c0 < nkc; c0 += 32) {
      int h[32];
#pragma unroll
      for (int q = 0; q < 32; ++q) h[q] = (c0 + q < nkc) ? ld_coh(P.hist + (size_t)(c0 + q) * E + e) : 0;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        base += c0 + q < c ? h[q] : 0;
        total += h[q];
      }
    }
    sm.u.r.scan1[e] = base;
    sm.u.r.hist[e] = total;  // (the chunk's own counts there are no longer needed)
    sm.u.r.tmp[e] = (total + P.bm - 1) / P.bm;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  if (wave == 0) wave_excl_scan(sm.u.r.hist, sm.u.r.scan0, E, lane);
  if (wave == 1) wave_excl_scan(sm.u.r.tmp, sm.u.r.mto, E, lane);
  __syncthreads();
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  chunk_scatter(P, c, ntok, sm.u.r.scan0, sm.u.r.scan1, sm.u.r.mto, sm);
}

template <int WT> struct ActT { using type = uint16_t; };
template <> struct ActT<WF32> { using type = float; };

// 4 consecutive values of H or Y (device-coherent: read by other workgroups)
template <int WT>
__device__ __forceinline__ void store4(void *base, size_t idx, f4 v) {
  if constexpr (WT == WF32) {
    float *p = reinterpret_cast<float *>(base) + idx;
    st_coh64(p, (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32));
    st_coh64(p + 2, (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32));
  } else {
    const uint64_t u = (uint64_t)f2bf(v[0]) | ((uint64_t)f2bf(v[1]) << 16) | ((uint64_t)f2bf(v[2]) << 32) |
                       ((uint64_t)f2bf(v[3]) << 48);
    st_coh64(reinterpret_cast<uint16_t *>(base) + idx, u);
  }
}

// The result tile of one wave (NC fragments of 16 columns by MG groups of 16 rows; lane
// (g, j) holds columns 16 c + 4 g .. 16 c + 4 g + 3 of row 16 b + j in v[c][b]) stored to rows
// [0, m) of a row-major matrix in the activation dtype, through the wave's slab of LDS: each
// row's 16 * NC values leave as one contiguous run, 16 bytes per lane per store, rather than
// as 8-byte pieces scattered over four times as many lines.  base: the tile's first row (a
// buffer resource: the rows' offsets from it stay below 4 GB, every one being below the
// number of tokens times the row length), ld: row length in elements, col0: the wave's
// first column.  Device-coherent stores (read by other workgroups in this launch).  A wave
// reads back only what its own lanes wrote, and its LDS operations complete in order.
template <int WT, int NC, int NFT, int MG>
__device__ __forceinline__ void store_tile(const f4 (&v)[NFT][MG], char *slab, const void *base, int ld, int col0, int m) {
  constexpr int ES = WT == WF32 ? 4 : 2;
  constexpr int RB = NC * 16 * ES, RS = RB + 16, LPR = RB / 16, RPI = 64 / LPR;
  static_assert(NC <= NFT && RPI >= 1 && 16 % RPI == 0, "tile store shape");
  const int lane = otid() & 63, g = lane >> 4, j = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base);
  const int rr = lane / LPR, cb = (lane % LPR) * 16;
#pragma unroll
  for (int b = 0; b < MG; ++b) {
    if (b * 16 >= m) break;
#pragma unroll
    for (int a = 0; a < NC; ++a) {
      char *p = slab + j * RS + (16 * a + 4 * g) * ES;
      if constexpr (ES == 4) {
        *reinterpret_cast<f4 *>(p) = v[a][b];
      } else {
        const uint32_t lo = (uint32_t)f2bf(v[a][b][0]) | ((uint32_t)f2bf(v[a][b][1]) << 16);
        const uint32_t hi = (uint32_t)f2bf(v[a][b][2]) | ((uint32_t)f2bf(v[a][b][3]) << 16);
        *reinterpret_cast<uint2 *>(p) = make_uint2(lo, hi);
      }
    }
#pragma unroll
    for (int q = 0; q < 16 / RPI; ++q) {
      const int row = q * RPI + rr;
      const u32x4 x = *reinterpret_cast<const u32x4 *>(slab + row * RS + cb);
      if (b * 16 + row < m)  // (unsigned: the offset may pass 2 GB, never 4 GB)
        __builtin_amdgcn_raw_buffer_store_b128(
            x, rs, ((uint32_t)(b * 16 + row) * (uint32_t)ld + (uint32_t)col0) * (uint32_t)ES + (uint32_t)cb, 0, kCpolSc1);
    }
  }
}
template <int WT, int NC, class SM>
__device__ __forceinline__ char *store_slab(SM &sm) {
  constexpr int ES = WT == WF32 ? 4 : 2, RS = NC * 16 * ES + 16;
  static_assert(sizeof(sm.u) >= kWaves * 16 * RS, "tile store slabs");
  return reinterpret_cast<char *>(&sm.u) + (otid() >> 6) * 16 * RS;
}

// gate/up item: rows (tokens) of one m-tile x gu_cols H columns; SwiGLU in registers
// pend: the completion counter of the workgroup's previous item still to be incremented
// (null: none); the item increments it once its own first loads are issued, and leaves its
// own counter in pend (the caller increments it before anything waits)
template <int WT, int MG, class SM>
__device__ __forceinline__ void gateup_item(const KParams &P, bool shared, int i, SM &sm, const Lds3 &lb,
                                            int *&pend) {
  using C = Core<WT, MG>;
  constexpr int NF = C::NF, NH = NF / 2;
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int gm = i / P.nt_gu, nt = i % P.nt_gu;
  int e, row0, m, counter;
  size_t hrow0;
  if (shared) {
    e = P.E;
    row0 = gm * P.bm;
    m = min(P.bm, P.T - row0);
    hrow0 = (size_t)P.T * P.k + row0;
    counter = gm;
  } else {
    const int4 ds = ld_coh_int4(P.desc + gm);
    e = uni(ds.x);
    row0 = uni(ds.y);
    m = uni(ds.z);
    hrow0 = row0;
    counter = P.n_shmt + gm;
  }
  for (int r = tid; r < C::BMR; r += kThreads) {
    const int rr = min(r, m - 1);
    int tok = shared ? row0 + rr : ld_coh(P.perm + row0 + rr) / P.k;
    sm.rows[r] = min(max(tok, 0), P.T - 1);
  }
  __syncthreads();
  const size_t wsz = Ty<WT>::WSZ, asz = Ty<WT>::ASZ;
  const int n0 = nt * P.gu_cols + wv * NH * 16;
  const char *wgb = reinterpret_cast<const char *>(shared ? P.shg : P.wg);
  const char *wub = reinterpret_cast<const char *>(shared ? P.shu : P.wu);
  const size_t emat = shared ? 0 : (size_t)e * P.n * P.d * wsz;
  const char *wrow[NF];
  const float *sc[NF];
#pragma unroll
  for (int a = 0; a < NH; ++a) {
    wrow[a] = frag_ptr(wgb + emat, n0 + 16 * a, (size_t)P.d * wsz, lane);
    wrow[a + NH] = frag_ptr(wub + emat, n0 + 16 * a, (size_t)P.d * wsz, lane);
    sc[a] = sc[a + NH] = nullptr;
    if constexpr (is_fp8w(WT)) {
      const int nkb = P.d / 128;
      const size_t soff = (shared ? 0 : (size_t)e * (P.n / 128) * nkb) + (size_t)((n0 + 16 * a) / 128) * nkb;
      sc[a] = (shared ? P.shsg : P.sg) + soff;
      sc[a + NH] = (shared ? P.shsu : P.su) + soff;
    }
  }
  f4 acc[NF][MG];
  const int ngroups = (m + 15) >> 4;
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  int *const sig = pend;
  pend = nullptr;
  if constexpr (WT == WQ8) {
    // the hidden rows as E4M3 codes and block scales, written earlier in this launch
    C::template run<true, kWStep>(acc, wrow, sc, reinterpret_cast<const char *>(P.xq), (size_t)P.d, sm.rows, lb, P.d,
                                  ngroups, P.xs, P.xs_stride, sig);
  } else {
    C::template run<false, kWStep>(acc, wrow, sc, reinterpret_cast<const char *>(P.x), (size_t)P.d * asz, sm.rows,
                                   lb, P.d, ngroups, nullptr, 0, sig);
  }
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  if constexpr (WT == WQ8) {
    // H requantised in registers: the item's 128 H columns are one 128-wide block of every
    // row, so each row's scale is the largest |h| over the four waves (lanes j, j+16, j+32,
    // j+48 of a wave hold the row's 4 x 8 values; the waves meet in LDS); codes go to H, the
    // exponent (+ 127) to the row's byte of hs
    float *red = reinterpret_cast<float *>(&sm.u.red[0][0]);  // [kWaves][BMR]
#pragma unroll
    for (int b = 0; b < MG; ++b) {
      float mx = 0.f;
#pragma unroll
      for (int a = 0; a < NH; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[a][b][q] = silu_mul(acc[a][b][q], acc[a + NH][b][q]);
          mx = fmaxf(mx, fabsf(acc[a][b][q]));
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) red[wv * C::BMR + b * 16 + j] = mx;
    }
    __syncthreads();
    uint8_t *hq = reinterpret_cast<uint8_t *>(P.H);
#pragma unroll
    for (int b = 0; b < MG; ++b) {
      const int r = b * 16 + j;
      float amax = red[r];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, red[w * C::BMR + r]);
      const int se = fp8_scale_exp(amax);
      if (r < m) {
#pragma unroll
        for (int a = 0; a < NH; ++a)
          st_coh(reinterpret_cast<int *>(hq + (hrow0 + r) * (size_t)P.n + n0 + 16 * a + 4 * g),
                 (int)fp8x4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3], se));
        if (wv == 0 && g == 0) st_coh8(P.hs + (hrow0 + r) * (size_t)P.hs_stride + nt, (uint32_t)(se + 127));
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < MG; ++b)
#pragma unroll
      for (int a = 0; a < NH; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[a][b][q] = silu_mul(acc[a][b][q], acc[a + NH][b][q]);
    store_tile<WT, NH>(acc, store_slab<WT, NH>(sm),
                       reinterpret_cast<const char *>(P.H) + hrow0 * (size_t)P.n * asz, P.n, n0, m);
  }
  pend = P.gudone + counter;  // (incremented once the H stores have completed)
}

// down item: rows of one m-tile x dn_cols output columns
// (pend: as for gateup_item)
template <int WT, int MG, class SM>
__device__ __forceinline__ bool down_item(const KParams &P, int i, SM &sm, const Lds3 &lb, int *&pend) {
  using C = Core<WT, MG>;
  constexpr int NF = C::NF;
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int gm = i / P.nt_dn, dt = i % P.nt_dn;
  if (!wg_wait_flush(P.gudone + gm, P.nt_gu, P.ctrl + kSlotInts * C_ERR, sm, pend)) return false;
  const bool shared = gm < P.n_shmt;
  int e, m;
  size_t row0;
  if (shared) {
    e = P.E;
    const int t0 = gm * P.bm;
    m = min(P.bm, P.T - t0);
    row0 = (size_t)P.T * P.k + t0;
  } else {
    const int4 ds = ld_coh_int4(P.desc + gm - P.n_shmt);
    e = uni(ds.x);
    row0 = (size_t)uni(ds.y);
    m = uni(ds.z);
  }
  for (int r = tid; r < C::BMR; r += kThreads) sm.rows[r] = (int)(row0 + min(r, m - 1));
  __syncthreads();
  const size_t wsz = Ty<WT>::WSZ, asz = Ty<WT>::ASZ;
  const int d0 = dt * P.dn_cols + wv * NF * 16;
  const char *wdb = reinterpret_cast<const char *>(shared ? P.shd : P.wd);
  const size_t emat = shared ? 0 : (size_t)e * P.d * P.n * wsz;
  const char *wrow[NF];
  const float *sc[NF];
#pragma unroll
  for (int a = 0; a < NF; ++a) {
    wrow[a] = frag_ptr(wdb + emat, min(d0 + 16 * a, P.d - 16), (size_t)P.n * wsz, lane);
    sc[a] = nullptr;
    if constexpr (is_fp8w(WT)) {
      const int nkb = P.n / 128;
      const float *sb = (shared ? P.shsd : P.sd) + (shared ? 0 : (size_t)e * (P.d / 128) * nkb);
      sc[a] = sb + (size_t)(min(d0 + 16 * a, P.d - 1) / 128) * nkb;
    }
  }
  f4 acc[NF][MG];
  const int ngroups = (m + 15) >> 4;
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  int *const sig = pend;
  pend = nullptr;
  if constexpr (WT == WQ8)  // H as E4M3 codes (one byte per value) and block scales
    C::template run<true, kWStep>(acc, wrow, sc, reinterpret_cast<const char *>(P.H), (size_t)P.n, sm.rows, lb, P.n,
                                  ngroups, P.hs, P.hs_stride, sig);
  else
    C::template run<true, kWStep>(acc, wrow, sc, reinterpret_cast<const char *>(P.H), (size_t)P.n * asz, sm.rows, lb,
                                  P.n, ngroups, nullptr, 0, sig);
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  // (d is a multiple of 256, the columns of a down item: every wave's columns exist)
  const size_t ysz = WT == WF32 ? 4 : 2;  // Y in the activation dtype (bf16 also with fp8 activations)
  store_tile<WT, NF>(acc, store_slab<WT, NF>(sm), reinterpret_cast<const char *>(P.Y) + row0 * (size_t)P.d * ysz,
                     P.d, d0, m);
  pend = P.dndone + gm;  // (incremented once the Y stores have completed)
  return true;
}

// ---------------------------------------------------------------------------------
// small m-tiles (at most 16 rows per expert, decode-sized problems): finer work units
// streamed straight from HBM to registers, so the weight stream is spread evenly over
// every workgroup and no unit waits for a long one.  A gate/up unit is 16 H columns
// (wave w: the gate (w < 2) or up fragment over one half of K, the halves added in a
// fixed order through LDS); a down unit is 128 output channels (wave w: 32 of them, two
// adjacent fragments, over all of K).  Token rows past the tile's end repeat its last row
// (the same addresses, so the loads coalesce) and are never stored.
// ---------------------------------------------------------------------------------

// acc[f] of NFR 16-row weight fragments against the same 16 token rows over nsteps
// 64-byte weight steps.  w[f]: this lane's weight bytes (row j, k-group g) at the first
// step; mk_a(): this lane's activation bytes for the same K positions (astep bytes per
// step), evaluated after the first weight loads are issued, so that a lookup it depends on
// (issued by the caller before) overlaps them.  D steps of loads stay in flight.  The loop
// body has no branches: steps past the end load one fixed line and multiply a zeroed
// activation, so every step issues the same memory operations; the first D steps are
// peeled so that the loads pending at the loop head are always in the same (interleaved)
// order, and the compiler can wait for exactly the step it consumes.  fp8: every two
// steps (128 K) close a scale block, whose partial sum is scaled by sc[f][block] before
// joining the result.
template <int WT, bool ACOH, int NFR, int D, class MkA>
__device__ __forceinline__ void stream_frags(f4 (&acc)[NFR], const char *const (&w)[NFR], MkA mk_a, int astep,
                                             int nsteps, const float *const (&sc)[NFR]) {
  constexpr int NA = WT == WFP8 ? 2 : 1;  // 16-byte activation loads per step
  const char *wdummy = reinterpret_cast<const char *>(uni64(reinterpret_cast<uint64_t>(w[0])));
  // fp8 block scales: lane l holds the scales of blocks l and l + 64 (read back with
  // readlane), so the loop issues no memory operation besides the stream itself
  const int nblk = nsteps >> 1;
  float scl0[NFR], scl1[NFR];
#pragma unroll
  for (int f = 0; f < NFR; ++f) {
    scl0[f] = scl1[f] = 0.f;
    if constexpr (WT == WFP8) {
      const int lane = otid() & 63;
      scl0[f] = sc[f][min(lane, nblk - 1)];
      scl1[f] = sc[f][min(lane + 64, nblk - 1)];
    }
  }
  uint4 wq[D][NFR], aq[D][NA];
  auto load_w = [&](int slot, int t) {
#pragma unroll
    for (int f = 0; f < NFR; ++f) wq[slot][f] = ld_stream16(t < nsteps ? w[f] + (size_t)t * kWStep : wdummy);
  };
#pragma unroll
  for (int u = 0; u < D; ++u) {
    load_w(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  const char *a = mk_a();
  const char *adummy = reinterpret_cast<const char *>(uni64(reinterpret_cast<uint64_t>(a)));
  auto load_a = [&](int slot, int t) {
#pragma unroll
    for (int x = 0; x < NA; ++x) {
      const char *ap = t < nsteps ? a + (size_t)t * astep + x * 16 : adummy;
      if constexpr (ACOH) aq[slot][x] = ld_coh16(ap);
      else aq[slot][x] = ld_glob16(ap);
    }
  };
#pragma unroll
  for (int u = 0; u < D; ++u) {
    load_a(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  f4 blk[NFR];
#pragma unroll
  for (int f = 0; f < NFR; ++f) acc[f] = blk[f] = f4{0.f, 0.f, 0.f, 0.f};
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
  auto step = [&](int t, int u) {
    const bool real = t + u < nsteps;
    const uint4 a0 = real ? aq[u][0] : z4, a1 = real ? aq[u][NA - 1] : z4;
#pragma unroll
    for (int f = 0; f < NFR; ++f) {
      if constexpr (WT == WFP8) {
        blk[f] = mfma_step<WT>(wq[u][f], a0, a1, blk[f]);
        if (u & 1) {
          const int b = min((t + u) >> 1, nblk - 1);
          const float scb =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(b < 64 ? scl0[f] : scl1[f]), b & 63));
          acc[f] += blk[f] * scb;
          blk[f] = f4{0.f, 0.f, 0.f, 0.f};
        }
      } else {
        acc[f] = mfma_step<WT>(wq[u][f], a0, a0, acc[f]);
      }
    }
    // refill the slot right behind the step it served (D steps in flight at all times)
    load_w(u, t + u + D);
    load_a(u, t + u + D);
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int u = 0; u < D; ++u) step(0, u);  // peeled first block
  for (int t = D; t < nsteps; t += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) step(t, u);
  }
}

// byte offset of lane k-group g's activation elements within one weight step
template <int WT> __device__ __forceinline__ int act_lane_off(int g) {
  if constexpr (WT == WFP8) return g * 32;  // 16 fp8 weights -> 16 bf16 activations (2 x 16 B)
  else return g * 16;                       // 16 bytes of the same element width
}

// gate/up unit (16-row m-tiles): 16 tokens x 16 H columns; waves 0/1 stream the 16 gate
// rows, waves 2/3 the 16 up rows, each over one half of K; the four partial tiles meet in
// LDS and wave 0 applies SwiGLU.  Shared-expert units need no routing, so they run in the
// first phase, while the router and top-k items are still working.
template <int WT, class SM>
__device__ __forceinline__ void gateup_unit(const KParams &P, bool shared, int i, SM &sm, bool deep) {
  constexpr int WSZ = Ty<WT>::WSZ, ASZ = Ty<WT>::ASZ, KU = Ty<WT>::KU;
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int gm = i / P.nt_gu, s = i % P.nt_gu;
  int e, row0, m, counter, tokr = 0;
  size_t hrow0;
  if (shared) {
    e = P.E;
    row0 = gm * 16;
    m = min(16, P.T - row0);
    hrow0 = (size_t)P.T * P.k + row0;
    counter = gm;
  } else {
    // the descriptor and the m-tile's token ids are independent loads (one round trip);
    // the token is consumed after the first weight loads are issued (stream_frag's mk_a)
    const int4 ds = ld_coh_int4(P.desc + gm);
    tokr = ld_coh(P.mtok + gm * 16 + j);
    __builtin_amdgcn_sched_barrier(0);
    e = uni(ds.x);
    row0 = uni(ds.y);
    m = uni(ds.z);
    hrow0 = row0;
    counter = P.n_shmt + gm;
  }
  const int rr = min(j, m - 1);
  const int kh = P.d / 2, k0 = (wv & 1) * kh;
  const void *wm = wv < 2 ? (shared ? P.shg : P.wg) : (shared ? P.shu : P.wu);
  const size_t emat = shared ? 0 : (size_t)e * P.n * P.d * WSZ;
  const char *w = frag_ptr(reinterpret_cast<const char *>(wm) + emat, 16 * s, (size_t)P.d * WSZ, lane) +
                  (size_t)(k0 * WSZ / 64) * kWStep;
  auto mk_a = [&]() {
    const int tok = min(max(shared ? row0 + rr : tokr, 0), P.T - 1);
    return reinterpret_cast<const char *>(P.x) + ((size_t)tok * P.d + k0) * ASZ + act_lane_off<WT>(g);
  };
  const float *sc[1] = {nullptr};
  if constexpr (WT == WFP8) {
    const int nkb = P.d / 128;
    sc[0] = (wv < 2 ? (shared ? P.shsg : P.sg) : (shared ? P.shsu : P.su)) +
            (shared ? 0 : (size_t)e * (P.n / 128) * nkb) + (size_t)((16 * s) / 128) * nkb + k0 / 128;
  }
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  const char *wf[1] = {w};
  f4 pa[1];
  if (deep) stream_frags<WT, false, 1, 8>(pa, wf, mk_a, KU * ASZ, kh / KU, sc);
  else stream_frags<WT, false, 1, 4>(pa, wf, mk_a, KU * ASZ, kh / KU, sc);
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  sm.u.red[wv][lane] = pa[0];
  __syncthreads();
  if (wv == 0 && j < m) {
    const f4 gs = sm.u.red[0][lane] + sm.u.red[1][lane];
    const f4 us = sm.u.red[2][lane] + sm.u.red[3][lane];
    f4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = silu_mul(gs[q], us[q]);
    store4<WT>(P.H, (hrow0 + j) * (size_t)P.n + 16 * s + 4 * g, h);
  }
  wg_signal(P.gudone + counter);
}

// down unit (16-row m-tiles): 128 output channels; each wave streams two adjacent 16-row
// fragments (32 channels, one contiguous stretch of the packed matrix) over the whole of n
template <int WT, class SM>
__device__ __forceinline__ bool down_unit(const KParams &P, int i, SM &sm, bool deep) {
  constexpr int WSZ = Ty<WT>::WSZ, ASZ = Ty<WT>::ASZ, KU = Ty<WT>::KU;
  const int tid = otid(), wv = uni(tid >> 6), lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int gm = i / P.nt_dn, ob = i % P.nt_dn;
  if (!wg_wait(P.gudone + gm, P.nt_gu, P.ctrl + kSlotInts * C_ERR, sm)) return false;
  const bool shared = gm < P.n_shmt;
  int e, m;
  size_t hrow0;
  if (shared) {
    e = P.E;
    const int t0 = gm * 16;
    m = min(16, P.T - t0);
    hrow0 = (size_t)P.T * P.k + t0;
  } else {
    const int4 ds = ld_coh_int4(P.desc + gm - P.n_shmt);
    e = uni(ds.x);
    hrow0 = (size_t)uni(ds.y);
    m = uni(ds.z);
  }
  const int o0 = ob * 128 + wv * 32;  // this wave's 32 output channels
  const char *wb = reinterpret_cast<const char *>(shared ? P.shd : P.wd) + (shared ? 0 : (size_t)e * P.d * P.n * WSZ);
  const char *w[2] = {frag_ptr(wb, o0, (size_t)P.n * WSZ, lane), frag_ptr(wb, o0 + 16, (size_t)P.n * WSZ, lane)};
  auto mk_a = [&]() {
    return reinterpret_cast<const char *>(P.H) + (hrow0 + min(j, m - 1)) * (size_t)P.n * ASZ + act_lane_off<WT>(g);
  };
  const float *sc[2] = {nullptr, nullptr};
  if constexpr (WT == WFP8) {
    const int nkb = P.n / 128;
    sc[0] = sc[1] = (shared ? P.shsd : P.sd) + (shared ? 0 : (size_t)e * (P.d / 128) * nkb) + (size_t)(o0 / 128) * nkb;
  }
  if (P.trace && tid == 0) sm.mark[0] = (uint32_t)wall_clock64();
  f4 acc[2];
  stream_frags<WT, true, 2, 4>(acc, w, mk_a, KU * ASZ, P.n / KU, sc);
  if (P.trace && tid == 0) sm.mark[1] = (uint32_t)wall_clock64();
  if (j < m) {
    store4<WT>(P.Y, (hrow0 + j) * (size_t)P.d + o0 + 4 * g, acc[0]);
    store4<WT>(P.Y, (hrow0 + j) * (size_t)P.d + o0 + 16 + 4 * g, acc[1]);
  }
  wg_signal(P.dndone + gm);
  return true;
}

// Waits (all threads) until the down items of every m-tile holding a row of combine item c
// (its tokens' k slots and the shared expert's row) are done.  False on timeout or fault.
template <class SM>
__device__ __forceinline__ bool combine_ready(const KParams &P, int c, SM &sm) {
  const int tid = otid(), k = P.k;
  const int t0 = c * P.ctok, ntok = min(P.ctok, P.T - t0), nsl = ntok * k;
  int *err = P.ctrl + kSlotInts * C_ERR;
  bool ok = true;
  for (int q = tid; q < nsl + (P.S ? ntok : 0); q += kThreads) {
    const int gm = q < nsl ? P.n_shmt + ld_coh(P.slotmt + (size_t)t0 * k + q) : (t0 + q - nsl) / P.bm;
    const int *ctr = P.dndone + min(max(gm, 0), P.mt_cap - 1);
    if (ld_relaxed(ctr) < P.nt_dn && !spin_geq(ctr, P.nt_dn, err, true)) ok = false;
  }
  if (tid == 0) sm.bcast[1] = 1;
  __syncthreads();
  if (!ok) sm.bcast[1] = 0;
  __syncthreads();
  return uni(sm.bcast[1]) != 0;
}

// combine: out[t] = sum_j w[t,j] * Y[inv_perm[t*k+j]] (+ Y[T*k + t]), float32, slot order.
// It ends the layer, so latency matters.  The item's gate weights and Y row indices (final
// once the scatter is done) are staged in LDS while it waits for the down items; then each
// thread takes UN (token, column) pairs at a time and issues the loads of all their Y rows,
// 8 slots per batch (and the shared expert's row with the last batch), before adding any.
// False on timeout or fault.
template <int WT, int UN, class SM>
__device__ __forceinline__ bool combine_item(const KParams &P, int c, SM &sm) {
  using A = typename ActT<WT>::type;
  constexpr int VEC = 16 / sizeof(A);
  constexpr int SB = 8;  // slots per batch
  const int tid = otid();
  const int t0 = c * P.ctok, ntok = min(P.ctok, P.T - t0);
  const int nv = P.d / VEC, k = P.k, npair = ntok * nv, nsl = ntok * k;
  const A *Y = reinterpret_cast<const A *>(P.Y);
  A *out = reinterpret_cast<A *>(P.out);
  static_assert(sizeof(sm.u) >= 8 * kMaxCombineSlots, "combine tables");
  float *sw = reinterpret_cast<float *>(&sm.u);
  int *sp = reinterpret_cast<int *>(sw + kMaxCombineSlots);
  for (int q = tid; q < nsl; q += kThreads) {
    sw[q] = ld_coh(P.wts + (size_t)t0 * k + q);
    sp[q] = min(max(ld_coh(P.inv_perm + (size_t)t0 * k + q), 0), P.T * k - 1);
  }
  if (!combine_ready(P, c, sm)) return false;  // (its barriers also publish the tables)
  auto add = [&](float (&acc)[VEC], const uint4 &raw, float w) {
    if constexpr (WT == WF32) {
      const float *f = reinterpret_cast<const float *>(&raw);
#pragma unroll
      for (int z = 0; z < VEC; ++z) acc[z] += w * f[z];
    } else {
      const uint16_t *h = reinterpret_cast<const uint16_t *>(&raw);
#pragma unroll
      for (int z = 0; z < VEC; ++z) acc[z] += w * bf2f(h[z]);
    }
  };
  for (int q0 = tid; q0 < npair; q0 += UN * kThreads) {
    int tl[UN], v[UN];
    float acc[UN][VEC];
#pragma unroll
    for (int x = 0; x < UN; ++x) {
      const int q = min(q0 + x * kThreads, npair - 1);  // (clamped: repeats a valid pair)
      tl[x] = q / nv;
      v[x] = q % nv;
#pragma unroll
      for (int z = 0; z < VEC; ++z) acc[x][z] = 0.f;
    }
    for (int j0 = 0; j0 < k; j0 += SB) {
      const bool last = j0 + SB >= k;
      uint4 raw[UN][SB], sh[UN];
      float w[UN][SB];
#pragma unroll
      for (int x = 0; x < UN; ++x)
#pragma unroll
        for (int b = 0; b < SB; ++b) {
          const int sl = tl[x] * k + min(j0 + b, k - 1);
          w[x][b] = sw[sl];
          raw[x][b] = ld_coh16(Y + (size_t)sp[sl] * P.d + v[x] * VEC);
        }
      if (P.S && last) {
#pragma unroll
        for (int x = 0; x < UN; ++x) sh[x] = ld_coh16(Y + ((size_t)P.T * k + t0 + tl[x]) * P.d + v[x] * VEC);
      }
#pragma unroll
      for (int x = 0; x < UN; ++x)
#pragma unroll
        for (int b = 0; b < SB; ++b)
          if (j0 + b < k) add(acc[x], raw[x][b], w[x][b]);
      if (P.S && last) {
#pragma unroll
        for (int x = 0; x < UN; ++x) add(acc[x], sh[x], 1.0f);
      }
    }
#pragma unroll
    for (int x = 0; x < UN; ++x) {
      if (q0 + x * kThreads >= npair) continue;
      uint4 o;
      if constexpr (WT == WF32) {
        o = make_uint4(__float_as_uint(acc[x][0]), __float_as_uint(acc[x][1]), __float_as_uint(acc[x][2]),
                       __float_as_uint(acc[x][3]));
      } else {
        uint32_t wv[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) wv[z] = (uint32_t)f2bf(acc[x][2 * z]) | ((uint32_t)f2bf(acc[x][2 * z + 1]) << 16);
        o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      *reinterpret_cast<uint4 *>(out + (size_t)(t0 + tl[x]) * P.d + v[x] * VEC) = o;
    }
  }
  return true;
}

// ---------------------------------------------------------------------------------
// the persistent kernel
// ---------------------------------------------------------------------------------

// register budget per kernel (waves per SIMD): 2 for the narrow tiles, 1 for the widest
template <int WT, int MG> struct Occ {
  static constexpr int waves = MG == 1 ? (WT == WFP8 ? 2 : 3) : (MG >= 8 || (MG == 4 && WT != WBF16)) ? 1 : 2;
};
// block scales of the tile's rows (WQ8): at most 256 blocks (d <= 32768) per row
template <int WT, int MG> struct ScaleBuf {
  static constexpr int BYTES = WT == WQ8 ? MG * 16 * 256 : 16;
};

template <int WT, int MG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occ<WT, MG>::waves)))
void moe_persistent(KParams P) {
  __shared__ Smem<WT, MG> sm;
  __shared__ __attribute__((aligned(16))) char act0[ActBuf<WT, MG>::BYTES];
  __shared__ __attribute__((aligned(16))) char act1[ActBuf<WT, MG>::BYTES];
  __shared__ __attribute__((aligned(16))) char act2[ActBuf<WT, MG>::BYTES2];
  __shared__ __attribute__((aligned(16))) char act3[Shape<WT, MG>::NBUF >= 4 ? ActBuf<WT, MG>::BYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t scl[ScaleBuf<WT, MG>::BYTES];
  const Lds3 lb{act0, act1, act2, act3, scl};
  static_assert(sizeof(Smem<WT, MG>) + 2 * ActBuf<WT, MG>::BYTES + ActBuf<WT, MG>::BYTES2 + sizeof(act3) +
                        ScaleBuf<WT, MG>::BYTES + 64 <= 160 * 1024,
                "LDS of one workgroup above the 160 KB of a CU");
  const int tid = threadIdx.x;
  int *ctrl = P.ctrl;
  int *err = ctrl + kSlotInts * C_ERR;
  // (a plain load: the magic word only changes between launches, and a cached read keeps
  // the whole grid from converging on one address at start-up)
  if (*reinterpret_cast<const volatile int *>(ctrl + kSlotInts * C_MAGIC) != kMagic) {
    if (tid == 0) __hip_atomic_store(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int n_Z = P.n_Z, n_L = P.n_L, n_K = P.n_K, n_SG = P.n_SG, n_S = P.n_S;
  const int n_Q = WT == WQ8 ? P.n_Q : 0;
  const int n_bound = n_Z + n_L;  // items before the first ticketed one (trace numbering)
  const int n_early = n_K + n_SG + n_S + n_Q;  // ticketed items before the gate/up, down, combine items
  const bool dyn = (P.phases & (PH_FFN | PH_COMBINE)) != 0;
  bool zero_seen = false, logits_seen = false, scat_seen = false, comb_scat_seen = false;
  bool quant_seen = WT != WQ8;
  // the combine needs the whole scatter: the S items, or the last K item's for one chunk
  const int n_S_comb = n_S + ((P.n_kc <= 1 && (P.phases & PH_PERMUTE)) ? 1 : 0);
  int n_mt = -1;
  int step = 0;
  // The completion counter of the last gate/up or down item of this workgroup (m-tiles above
  // 16 rows), incremented once its result stores complete: by the next item after its first
  // loads are issued (the stores drain while they are in flight), or here before anything
  // waits or the workgroup exits (what it waits for may depend on that counter).
  int *pend = nullptr;
  auto flush = [&]() {
    if (pend != nullptr) {
      wg_signal(pend);
      pend = nullptr;
    }
  };
  const bool dynamic = P.schedule == 0;
  // Dynamic tickets come from np = min(kTicketParts, grid) counters, one per partition of
  // the workgroups: partition p hands out the tickets p, p + np, ... in order.  Workgroup b
  // joins partition (b + b / 8) % np: the hardware deals workgroups to the 8 XCDs round
  // robin (b % 8), so every partition draws on all XCDs, and a partition that falls behind
  // near the end still has the whole chip's bandwidth; workgroup b < np joins partition b,
  // so every partition has a workgroup and every ticket a taker.  Device atomics on one
  // address serialise (~11 ns each), and every workgroup takes a ticket at start-up and one
  // per item: split over the partitions, neither the start-up burst nor the steady stream
  // of ticket atomics queues up behind one address.  A ticket is still only ever taken by a
  // running workgroup, and each partition's workgroups take their tickets in increasing
  // order while waiting only for smaller tickets, so every wait ends (induction over the
  // tickets, as with one counter).  Thread 0 keeps the next ticket prefetched, so the
  // atomic's latency overlaps the current item.
  const int nparts = min(kTicketParts, (int)gridDim.x), part = ((int)blockIdx.x + (int)blockIdx.x / 8) % nparts;
  int *pctr = ctrl + kSlotInts * (C_PTICKET + part);
  int next = 0;
  // item trace record (moe_forward_ex with a trace buffer); `item` numbers every item of the
  // launch, router items included, in phase order
  auto record = [&](int item, int kind, uint64_t t_start) {
    if (P.trace && tid == 0 && item < P.trace_cap) {
      unsigned long long *rec = P.trace + 4 * (size_t)item;
      rec[0] = t_start;
      rec[1] = wall_clock64();
      // item | tile-loop start and end (16-bit offsets from the item start, 10 ns units)
      const uint32_t m0 = sm.mark[0], m1 = sm.mark[1];
      const unsigned long long d0 = m0 ? min((uint32_t)(m0 - (uint32_t)t_start), 0xffffu) : 0;
      const unsigned long long d1 = m1 ? min((uint32_t)(m1 - (uint32_t)t_start), 0xffffu) : 0;
      rec[2] = (unsigned long long)(uint32_t)item | (d0 << 32) | (d1 << 48);
      rec[3] = ((unsigned long long)blockIdx.x << 32) | (unsigned)kind;
    }
  };
  // Router items take no ticket: workgroup b runs items b, b + grid, ... before its first
  // ticket.  They wait for nothing, so each finishes, and the first workgroups of the launch
  // start on them at once rather than after a ticket atomic of the start-up burst.
  for (int r = (int)blockIdx.x; r < n_L; r += (int)gridDim.x) {
    __syncthreads();
    const uint64_t t_start = P.trace ? wall_clock64() : 0;
    if (P.trace && tid == 0) sm.mark[0] = sm.mark[1] = 0;
    if constexpr (MG == 1) logits_item_split<WT>(P, r, sm);
    else logits_item_tile<WT, MG>(P, r, sm, lb);
    wg_signal(ctrl + kSlotInts * C_LDONE);
    record(n_Z + r, K_ROUTER, t_start);
  }
  // The first ticket is taken here, before the counter-clearing items, so that every
  // workgroup holds one top-k ticket before any workgroup takes a second ticket (a top-k
  // item behind another one on the same workgroup would delay the plan by a whole item).
  bool have_next = false;  // (thread 0) `next` holds a fetched ticket
  if (dynamic && tid == 0) {
    next = __hip_atomic_fetch_add(pctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    have_next = true;
  }
  // The counter-clearing items take no ticket either: workgroup grid - 1 - b runs items b,
  // b + grid, ... (the last workgroups, which have router items only when every one has).
  for (int z = (int)gridDim.x - 1 - (int)blockIdx.x; z < n_Z; z += (int)gridDim.x) {
    __syncthreads();
    const uint64_t t_start = P.trace ? wall_clock64() : 0;
    if (P.trace && tid == 0) sm.mark[0] = sm.mark[1] = 0;
    zero_item(P, z);
    wg_signal(ctrl + kSlotInts * C_ZDONE);
    record(z, K_ZERO, t_start);
  }
  // Late phase (m-tiles of more than 16 rows, dynamic schedule).  The gate/up and down items
  // are split over one queue per XCD: the m-tiles u (the shared expert's first, then the
  // routed ones, in expert order) form contiguous ranges, XCD x holding [x U / 8, (x+1) U / 8)
  // of the U m-tiles; workgroups start on the queue of the XCD they run on (hardware register
  // XCC_ID), so the items of one m-tile share their gathered token rows through that XCD's L2.
  // Within a queue the gate/up items come first, then the down items, each in groups of
  // group_m m-tiles taken n-tile by n-tile: consecutive items of a group read the same weight
  // rows when the group's m-tiles belong to one expert (an expert with more rows than an
  // m-tile), so its weights are fetched from HBM about once per group, as the grouped
  // ordering of the vLLM config page (section 03, GROUP_SIZE_M) does for one GEMM.  A
  // workgroup whose queue is empty takes items from the next XCD's queue, and so on, until
  // every queue is empty; only then does it take combine items (from its early partition's
  // counter, continuing with the ticket that ended its early items).  Every wait still ends:
  // a down item waits for gate/up items of its own m-tile, earlier in the same queue; a
  // combine item starts only after every gate/up and down item has been taken, by running
  // workgroups, and those wait for nothing later.
  int stage = 0;   // 0: early tickets; late phase: 1 per-XCD gate/up and down queues, 2 combine
  int held = 0;    // late phase: the workgroup's current early ticket (combine items)
  int xcc = 0, xq = -1, lnext = 0;  // late phase: this XCD, queues emptied so far, prefetched ticket
  for (;;) {
    __syncthreads();
    // the next item: phase 0 top-k, 1 shared gate/up, 2 scatter, 3 gate/up, 4 down, 5 combine
    int phase = -1, idx = 0, item = 0;
    if (stage == 0) {
      if (dynamic) {
        if (tid == 0) {
          if (!have_next) next = __hip_atomic_fetch_add(pctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          sm.bcast[0] = part + nparts * next;
        }
        __syncthreads();
      }
      const int ticket = dynamic ? uni(sm.bcast[0]) : (int)blockIdx.x + step * (int)gridDim.x;
      ++step;
      // prefetch the next ticket (its value is read at the top of the next iteration), except
      // during a top-k or quantisation item: a second ticket taken then could be another item
      // of the same phase, which this workgroup would start only after the current one, while
      // the phase's last item holds up the next phase
      have_next = false;
      const bool burst = ticket < n_K || (ticket >= n_K + n_SG && ticket < n_K + n_SG + n_Q);
      if (dynamic && tid == 0 && !burst) {
        next = __hip_atomic_fetch_add(pctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        have_next = true;
      }
      item = ticket + n_bound;  // (counter-clearing and router items are not ticketed)
      int i = ticket;
      if (i < n_K) {
        phase = 0, idx = i;
      } else if ((i -= n_K) < n_SG) {
        phase = 1, idx = i;
      } else if ((i -= n_SG) < n_Q) {
        phase = 6, idx = i;
      } else if ((i -= n_Q) < n_S) {
        phase = 2, idx = i;
      } else {
        i -= n_S;
        if (!dyn) break;
        if (MG > 1 && P.late) {  // (16-row m-tiles never use the late phase)
          held = ticket;
          stage = 1;
          continue;
        }
        if (n_mt < 0) flush();
        if (n_mt < 0 && (n_mt = wg_wait_plan(P, sm)) < 0) break;
        const int n_G = n_mt * P.nt_gu;
        const int n_D = (n_mt + P.n_shmt) * P.nt_dn;
        if (i < n_G) phase = 3, idx = i;
        else if ((i -= n_G) < n_D) phase = 4, idx = i;
        else if ((i -= n_D) < P.n_comb) phase = 5, idx = i;
        else break;
      }
    } else if (MG > 1 && stage == 1) {
      if (n_mt < 0) flush();
      if (n_mt < 0 && (n_mt = wg_wait_plan(P, sm)) < 0) break;
      const int U = P.n_shmt + n_mt;
      if (xq < 0) {  // first late item of this workgroup: its XCD's queue
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(xcc));
        xq = 0;
        if (tid == 0)
          lnext = __hip_atomic_fetch_add(ctrl + kSlotInts * (C_LTICKET + (xcc & (kXcds - 1))), 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
      const int x = (xcc + xq) & (kXcds - 1);
      const int lo = x * U / kXcds, hi = (x + 1) * U / kXcds, nu = hi - lo;
      const int nG = nu * P.nt_gu, nGD = nG + nu * P.nt_dn;
      if (tid == 0) sm.bcast[0] = lnext;
      __syncthreads();
      int q = uni(sm.bcast[0]);
      int *lctr = ctrl + kSlotInts * (C_LTICKET + x);
      if (q >= nGD) {  // this queue is empty: the next XCD's, and after the last, the combine
        if (++xq == kXcds) {
          stage = 2;
        } else if (tid == 0) {
          lnext = __hip_atomic_fetch_add(ctrl + kSlotInts * (C_LTICKET + ((xcc + xq) & (kXcds - 1))), 1,
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        continue;
      }
      if (tid == 0) lnext = __hip_atomic_fetch_add(lctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool gu = q < nG;
      if (!gu) q -= nG;
      // q -> (m-tile u, n-tile j): groups of group_m m-tiles, n-tile-major inside a group
      const int ntile = gu ? P.nt_gu : P.nt_dn, per = P.group_m * ntile;
      const int grp = q / per, r = q - grp * per, u0 = lo + grp * P.group_m, gs = min(P.group_m, hi - u0);
      const int j = r / gs, u = u0 + (r - j * gs);
      if (!gu) {
        phase = 4, idx = u * P.nt_dn + j;
        item = n_bound + n_early + U * P.nt_gu + idx;
      } else {
        phase = u < P.n_shmt ? 1 : 3;
        idx = (u < P.n_shmt ? u : u - P.n_shmt) * P.nt_gu + j;
        item = n_bound + n_early + u * P.nt_gu + j;
      }
    } else if (MG > 1) {
      // combine items: this workgroup's early tickets from `held` on, item = ticket - n_early
      const int c = held - n_early;
      if (c >= P.n_comb) break;
      if (tid == 0) {
        sm.bcast[0] = part + nparts * next;
        next = __hip_atomic_fetch_add(pctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
      held = uni(sm.bcast[0]);
      phase = 5, idx = c;
      item = n_bound + n_early + (P.n_shmt + n_mt) * (P.nt_gu + P.nt_dn) + c;
    } else {
      break;
    }
    const uint64_t t_start = P.trace ? wall_clock64() : 0;
    if (P.trace && tid == 0) sm.mark[0] = sm.mark[1] = 0;
    int kind = -1;
    const int i = idx;
    if (phase == 0) {
      if (!(P.phases & PH_IDS_GIVEN) && !logits_seen) {
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_LDONE, n_L, err, sm)) break;
        logits_seen = true;
      }
      if (!zero_seen && P.n_kc > 1) {  // chunk histograms are cleared by the Z items
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      topk_item<kMaxRouterSplit(is_fp8w(WT), MG)>(P, i, sm);
      kind = K_TOPK;
    } else if (phase == 1) {
      if (!zero_seen) {
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      if (!quant_seen) {  // the quantised hidden rows
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_QDONE, n_Q, err, sm)) break;
        quant_seen = true;
      }
      if constexpr (MG == 1) gateup_unit<WT>(P, true, i, sm, 2 * n_SG <= kWaves * (int)gridDim.x);
      else gateup_item<WT, MG>(P, true, i, sm, lb, pend);
      kind = K_SHGU;
    } else if (phase == 2) {
      // (the scatter needs the chunk histograms only, complete once every top-k item is)
      flush();
      if (!wg_wait(ctrl + kSlotInts * C_KDONE, n_K, err, sm)) break;
      scatter_item(P, i, sm);
      wg_signal(ctrl + kSlotInts * C_SDONE);
      kind = K_SCATTER;
    } else if (phase == 6) {
      if constexpr (WT == WQ8) {
        quant_item(P, i);
        wg_signal(ctrl + kSlotInts * C_QDONE);
      }
      kind = K_QUANT;
    } else if (phase == 3 || phase == 4) {
      // small-tile units: a deep prefetch (8 steps) when the units are too few to keep the
      // memory system busy, else a shallow one (4 steps): with every wave of the grid
      // streaming, more requests in flight only add contention
      const bool deep = 2 * n_mt * P.nt_gu <= kWaves * (int)gridDim.x;
      if (!scat_seen) {
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_SDONE, n_S, err, sm)) break;
        scat_seen = true;
      }
      if (!zero_seen) {  // the dependency counters must be cleared before they are used
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      if (phase == 3 && !quant_seen) {  // the quantised hidden rows
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_QDONE, n_Q, err, sm)) break;
        quant_seen = true;
      }
      if (phase == 3) {
        if constexpr (MG == 1) gateup_unit<WT>(P, false, i, sm, deep);
        else gateup_item<WT, MG>(P, false, i, sm, lb, pend);
        kind = K_GU;
      } else {
        if constexpr (MG == 1) {
          if (!down_unit<WT>(P, i, sm, deep)) break;
        } else {
          if (!down_item<WT, MG>(P, i, sm, lb, pend)) break;
        }
        kind = K_DN;
      }
    } else {
      // the token's rows of Y are final once the down items of their m-tiles are done (the
      // slot m-tiles come from the scatter; the counters are valid once cleared)
      if (!comb_scat_seen) {
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_SDONE, n_S_comb, err, sm)) break;
        comb_scat_seen = true;
      }
      if (!zero_seen) {
        flush();
        if (!wg_wait(ctrl + kSlotInts * C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      flush();
      if (!combine_item<WT, Occ<WT, MG>::waves == 1 ? 4 : kCombineUnroll>(P, i, sm)) break;
      kind = K_COMB;
    }
    record(item, kind, t_start);
  }
  // The last workgroup out resets the control block for the next call.  Thread 0 made every
  // counter update of this workgroup (the unused prefetched ticket included); once they have
  // all returned, a relaxed increment of the exit counter orders them before the reset.  No
  // acquire or release here: at agent scope those write back and invalidate the XCD's whole
  // L2, and with every workgroup leaving at the end that would stall the items still running.
  flush();
  __syncthreads();
  if (tid == 0) {
    wait_vm0();
    const int old = __hip_atomic_fetch_add(ctrl + kSlotInts * C_EXIT, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (int)gridDim.x - 1) {
      for (int s : {C_ZDONE, C_LDONE, C_KDONE, C_SDONE, C_QDONE, C_EXIT}) st_coh(ctrl + kSlotInts * s, 0);
      if (P.reset_err) st_coh(err, 0);
      for (int q = 0; q < kTicketParts; ++q) st_coh(ctrl + kSlotInts * (C_PTICKET + q), 0);
      for (int q = 0; q < kXcds; ++q) st_coh(ctrl + kSlotInts * (C_LTICKET + q), 0);
      for (int c = 0; c < kPlanCopies; ++c) st_coh(ctrl + plan_flag_word(c), 0);
    }
  }
}

__global__ void ws_init_kernel(int *ctrl, size_t nwords) {
  for (size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x; q < nwords; q += (size_t)gridDim.x * blockDim.x)
    ctrl[q] = (q == (size_t)kSlotInts * C_MAGIC) ? kMagic : 0;
}

// row-major -> packed fragment layout of nmat matrices of [R rows, C bytes] (R % 16 == 0,
// C % 64 == 0), contiguous in src and dst: one 16-byte chunk per thread, written in order
__global__ void pack_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst, size_t nchunks, int C16) {
  const size_t frag16 = (size_t)16 * C16;  // 16-byte chunks per fragment (16 rows)
  for (size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x; q < nchunks; q += (size_t)gridDim.x * blockDim.x) {
    const size_t f = q / frag16, rem = q % frag16;
    const int s = (int)(rem >> 6), l = (int)(rem & 63), j = l & 15, g = l >> 4;
    dst[q] = src[(f * 16 + j) * C16 + 4 * s + g];
  }
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------
typedef void (*KernelFn)(KParams);

template <int WT> KernelFn pick_kernel(int mg) {
  if constexpr (WT == WQ8) {  // (m-tiles above 16 rows only)
    return mg == 2 ? moe_persistent<WQ8, 2> : mg == 4 ? moe_persistent<WQ8, 4> : mg == 10 ? moe_persistent<WQ8, 10> : moe_persistent<WQ8, 8>;
  } else {
    switch (mg) {
      case 1: return moe_persistent<WT, 1>;
      case 2: return moe_persistent<WT, 2>;
      case 4: return moe_persistent<WT, 4>;
      default: break;
    }
    if (mg == 10) return moe_persistent<WT, 10>;
    return moe_persistent<WT, 8>;
  }
}

// kind: WF32, WBF16, WFP8 or WQ8 (fp8 weights and activations)
KernelFn kernel_for(int kind, int mg) {
  if (kind == WF32) return pick_kernel<WF32>(mg);
  if (kind == WBF16) return pick_kernel<WBF16>(mg);
  if (kind == WQ8) return pick_kernel<WQ8>(mg);
  return pick_kernel<WFP8>(mg);
}

int kernel_kind(const moe_problem *p, const Tiles &t) {
  if (p->w_dtype == MOE_F32) return WF32;
  if (p->w_dtype == MOE_BF16) return WBF16;
  return t.aq ? WQ8 : WFP8;
}

struct DevInfo {
  int cus = 0;
  int occ[4][5] = {};  // [kernel kind][m-tile size 16, 32, 64, 128, 160 rows]
};

std::mutex g_mu;
DevInfo g_dev[64];
bool g_have[64];

moe_status device_info(int dev, int kind, int mg, int *cus, int *occ) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dev < 0 || dev >= 64) return MOE_ERR_HIP;
  DevInfo &D = g_dev[dev];
  if (!g_have[dev]) {
    if (hipDeviceGetAttribute(&D.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
    g_have[dev] = true;
  }
  const int mi = mg == 1 ? 0 : mg == 2 ? 1 : mg == 4 ? 2 : mg == 8 ? 3 : 4;
  int &o = D.occ[kind][mi];
  if (o == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(kernel_for(kind, mg)),
                                                     kThreads, 0) != hipSuccess)
      return MOE_ERR_HIP;
    o = nb > 0 ? nb : 1;
  }
  *cus = D.cus;
  *occ = o;
  return MOE_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Call {
  const moe_problem *p;
  const void *hidden, *w_router;
  const float *bias;
  const moe_weights *w;
  void *out;
  int32_t *ids_user;
  float *wts_user, *logits_user;
  const int32_t *ids_in;
  int32_t *counts_user, *offsets_user, *perm_user, *invperm_user;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
  int phases;
  const moe_launch_options *opts;
  int reset_err;
};

moe_status launch(const Call &c) {
  const moe_problem *p = c.p;
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (!c.ws || (reinterpret_cast<uintptr_t>(c.ws) & 255u)) return MOE_ERR_INVALID_ARGUMENT;
  Tiles forced;
  bool have_forced = false;
  if (c.opts) {
    if (c.opts->schedule == 2) return MOE_ERR_UNSUPPORTED;
    if (c.opts->grid_wgs < 0 || c.opts->schedule < 0 || c.opts->schedule > 1) return MOE_ERR_INVALID_ARGUMENT;
    if (c.opts->trace_bytes < 0 || (c.opts->trace && !aligned16(c.opts->trace))) return MOE_ERR_INVALID_ARGUMENT;
    if (c.opts->m_tile_rows || c.opts->group_m) {
      if (!override_tiles(p, c.opts->m_tile_rows, c.opts->group_m, &forced)) return MOE_ERR_INVALID_ARGUMENT;
      have_forced = true;
    }
  }
  const Layout L = make_layout(p, have_forced ? &forced : nullptr);
  if (c.ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (p->T == 0) return MOE_OK;

  char *ws = static_cast<char *>(c.ws);
  KParams P{};
  P.T = (int)p->T;
  P.d = p->d;
  P.n = p->n;
  P.E = p->E;
  P.k = p->k;
  P.S = p->n_shared;
  P.phases = c.phases;
  P.bm = L.tiles.bm;
  P.tk = L.tiles.tk;
  P.gu_cols = L.tiles.gu_cols;
  P.dn_cols = L.tiles.dn_cols;
  P.n_lt = L.n_lt;
  P.n_le = L.n_le;
  P.kt_tok = L.kt_tok;
  P.rt_split = L.tiles.rt_split;
  P.n_kt = L.n_kt;
  P.n_kc = L.n_kc;
  P.n_shmt = L.n_shmt;
  P.nt_gu = L.nt_gu;
  P.nt_dn = L.nt_dn;
  P.n_comb = L.n_comb;
  P.ctok = L.tiles.ctok;
  P.mt_cap = L.mt_routed_max + L.n_shmt;
  P.x = c.hidden;
  P.wr = c.w_router;
  P.bias = c.bias;
  if (c.w) {
    P.wg = c.w->w_gate;
    P.wu = c.w->w_up;
    P.wd = c.w->w_down;
    P.sg = c.w->s_gate;
    P.su = c.w->s_up;
    P.sd = c.w->s_down;
    P.shg = c.w->sh_gate;
    P.shu = c.w->sh_up;
    P.shd = c.w->sh_down;
    P.shsg = c.w->sh_s_gate;
    P.shsu = c.w->sh_s_up;
    P.shsd = c.w->sh_s_down;
  }
  P.out = c.out;
  P.logits = c.logits_user ? c.logits_user : reinterpret_cast<float *>(ws + L.off_logits);
  P.lpart = reinterpret_cast<float *>(ws + L.off_lpart);
  P.ids = c.ids_user ? c.ids_user : (c.ids_in ? const_cast<int *>(c.ids_in) : reinterpret_cast<int *>(ws + L.off_ids));
  P.wts = c.wts_user ? c.wts_user : reinterpret_cast<float *>(ws + L.off_wts);
  P.counts = c.counts_user ? c.counts_user : reinterpret_cast<int *>(ws + L.off_counts);
  P.offsets = c.offsets_user ? c.offsets_user : reinterpret_cast<int *>(ws + L.off_offsets);
  P.perm = c.perm_user ? c.perm_user : reinterpret_cast<int *>(ws + L.off_perm);
  P.inv_perm = c.invperm_user ? c.invperm_user : reinterpret_cast<int *>(ws + L.off_invperm);
  P.ctrl = reinterpret_cast<int *>(ws);
  P.gudone = reinterpret_cast<int *>(ws + L.off_gudone);
  P.dndone = P.gudone + ctr_words(L);
  P.slotmt = reinterpret_cast<int *>(ws + L.off_slotmt);
  P.desc = reinterpret_cast<int4 *>(ws + L.off_desc);
  P.hist = reinterpret_cast<int *>(ws + L.off_hist);
  P.mtoff = reinterpret_cast<int *>(ws + L.off_mtoff);
  P.mtok = reinterpret_cast<int *>(ws + L.off_mtok);
  P.H = ws + L.off_h;
  P.Y = ws + L.off_y;
  P.aq = L.tiles.aq;
  P.xq = reinterpret_cast<uint8_t *>(ws + L.off_xq);
  P.xs = reinterpret_cast<uint8_t *>(ws + L.off_xs);
  P.hs = reinterpret_cast<uint8_t *>(ws + L.off_hs);
  P.xs_stride = L.xs_stride;
  P.hs_stride = L.hs_stride;
  if (c.opts && c.opts->trace) {
    P.trace = static_cast<unsigned long long *>(c.opts->trace);
    P.trace_cap = c.opts->trace_bytes / 32;
  }

  P.schedule = c.opts ? c.opts->schedule : 0;
  P.late = (L.tiles.late && P.schedule == 0 && (P.phases & PH_FFN)) ? 1 : 0;
  P.group_m = L.tiles.group_m;
  const PhaseCounts pc = phase_counts(L, P.phases, P.late != 0);
  P.n_Z = pc.z;
  P.n_L = pc.l;
  P.n_K = pc.k;
  P.n_SG = pc.sg;
  P.n_S = pc.s;
  P.n_Q = pc.q;
  P.gd_words = pc.gd_words;
  P.hist_words = pc.hist_words;
  int n_items = pc.z + pc.l + pc.q + pc.k + pc.sg + pc.s;
  if (P.phases & PH_FFN)
    n_items += L.mt_routed_max * (P.nt_gu + P.nt_dn) + P.n_shmt * P.nt_dn + P.n_comb + (P.late ? P.n_shmt * P.nt_gu : 0);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  int cus = 0, occ = 0;
  const int kind = kernel_kind(p, L.tiles);
  st = device_info(dev, kind, L.tiles.mg, &cus, &occ);
  if (st != MOE_OK) return st;
  int grid = cus * occ;
  if (c.opts && c.opts->grid_wgs > 0) grid = c.opts->grid_wgs;
  P.reset_err = c.reset_err;
  // never more workgroups than can be resident at once: the clearing and router items (and,
  // with the static schedule, every item) are bound to workgroups, so every workgroup of the
  // launch must be able to run while the others wait
  if (grid > cus * occ) grid = cus * occ;
  if (grid > n_items && P.schedule == 0) grid = n_items > 0 ? n_items : 1;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel_for(kind, L.tiles.mg), dim3(grid), dim3(kThreads), 0, c.stream, P);
  if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status check_weights(const moe_problem *p, const moe_weights *w) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(w->w_gate) || !aligned16(w->w_up) || !aligned16(w->w_down)) return MOE_ERR_INVALID_ARGUMENT;
  const bool fp8 = p->w_dtype == MOE_FP8_E4M3;
  if (fp8 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARGUMENT;
  if (p->n_shared) {
    if (!w->sh_gate || !w->sh_up || !w->sh_down) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w->sh_gate) || !aligned16(w->sh_up) || !aligned16(w->sh_down)) return MOE_ERR_INVALID_ARGUMENT;
    if (fp8 && (!w->sh_s_gate || !w->sh_s_up || !w->sh_s_down)) return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------
// the allocation-free entry point's workspace: a fixed array in device memory, one copy
// per GPU (each device that loads the library's code object holds its own, at its own
// address, until the process ends).  Host code never passes `scratch` itself to a kernel:
// on the host the name stands for a host-side shadow, not a device address; the device
// address comes from hipGetSymbolAddress, once per device, and only that is used.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch[64];  // device address of `scratch` on device i, once initialised

// The device address of this device's scratch (the current device).  The first call on a
// device looks the address up and enqueues, on `stream`, a fill kernel that puts the whole
// array in the state moe_workspace_init leaves a workspace in (a kernel, not a memset, so
// the call may be stream-captured).
moe_status device_scratch(hipStream_t stream, void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    const size_t nwords = (size_t)MOE_NOALLOC_SCRATCH_BYTES / 4;
    hipLaunchKernelGGL(ws_init_kernel, dim3(4096), dim3(256), 0, stream, static_cast<int *>(p), nwords);
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u) || ws_bytes < (size_t)kCtrlBytes) return MOE_ERR_INVALID_ARGUMENT;
  const size_t nwords = ws_bytes / 4;
  size_t blocks = (nwords + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(ws_init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<int *>(ws), nwords);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_route(const moe_problem *p, const void *hidden, const void *w_router, const float *bias,
                     int32_t *topk_ids, float *topk_weights, float *logits, void *ws, size_t ws_bytes,
                     hipStream_t stream) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // nothing to read or write; pointers may be NULL
  if (!hidden || !w_router || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(hidden) || !aligned16(w_router)) return MOE_ERR_INVALID_ARGUMENT;
  Call c{};
  c.p = p;
  c.hidden = hidden;
  c.w_router = w_router;
  c.bias = bias;
  c.ids_user = topk_ids;
  c.wts_user = topk_weights;
  c.logits_user = logits;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = stream;
  c.phases = PH_ROUTE;
  return launch(c);
}

moe_status moe_permute(const moe_problem *p, const int32_t *topk_ids, int32_t *counts, int32_t *offsets,
                       int32_t *perm, int32_t *inv_perm, void *ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // nothing to read or write; pointers may be NULL
  if (!topk_ids || !counts || !offsets || !perm || !inv_perm) return MOE_ERR_INVALID_ARGUMENT;
  Call c{};
  c.p = p;
  c.ids_in = topk_ids;
  c.counts_user = counts;
  c.offsets_user = offsets;
  c.perm_user = perm;
  c.invperm_user = inv_perm;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = stream;
  c.phases = PH_PERMUTE | PH_IDS_GIVEN;
  return launch(c);
}

moe_status moe_forward_ex(const moe_problem *p, const void *hidden, const void *w_router, const float *bias,
                          const moe_weights *w, void *out, const moe_route_out *ro, void *ws, size_t ws_bytes,
                          hipStream_t stream, const moe_launch_options *opts) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;  // nothing to read or write; pointers may be NULL
  if (!hidden || !w_router || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(hidden) || !aligned16(w_router) || !aligned16(out)) return MOE_ERR_INVALID_ARGUMENT;
  if (out == hidden) return MOE_ERR_INVALID_ARGUMENT;
  if (p->w_layout != MOE_W_PACKED) return MOE_ERR_UNSUPPORTED;  // see moe_pack_weights
  st = check_weights(p, w);
  if (st != MOE_OK) return st;
  Call c{};
  c.p = p;
  c.hidden = hidden;
  c.w_router = w_router;
  c.bias = bias;
  c.w = w;
  c.out = out;
  if (ro) {
    c.ids_user = ro->topk_ids;
    c.wts_user = ro->topk_weights;
    c.logits_user = ro->logits;
    c.counts_user = ro->counts;
    c.offsets_user = ro->offsets;
    c.perm_user = ro->perm;
    c.invperm_user = ro->inv_perm;
  }
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = stream;
  c.phases = PH_ROUTE | PH_PERMUTE | PH_FFN | PH_COMBINE;
  c.opts = opts;
  return launch(c);
}

moe_status moe_forward(const moe_problem *p, const void *hidden, const void *w_router, const float *bias,
                       const moe_weights *w, void *out, const moe_route_out *ro, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  return moe_forward_ex(p, hidden, w_router, bias, w, out, ro, ws, ws_bytes, stream, nullptr);
}

moe_status moe_forward_noalloc(const moe_problem *p, const void *hidden, const void *w_router, const float *bias,
                               const moe_weights *w, void *out, const moe_route_out *ro, hipStream_t stream) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (make_layout(p).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (p->T == 0) return MOE_OK;  // nothing to read or write; pointers may be NULL
  if (!hidden || !w_router || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(hidden) || !aligned16(w_router) || !aligned16(out)) return MOE_ERR_INVALID_ARGUMENT;
  if (out == hidden) return MOE_ERR_INVALID_ARGUMENT;
  if (p->w_layout != MOE_W_PACKED) return MOE_ERR_UNSUPPORTED;
  st = check_weights(p, w);
  if (st != MOE_OK) return st;
  void *ws = nullptr;
  st = device_scratch(stream, &ws);
  if (st != MOE_OK) return st;
  Call c{};
  c.p = p;
  c.hidden = hidden;
  c.w_router = w_router;
  c.bias = bias;
  c.w = w;
  c.out = out;
  if (ro) {
    c.ids_user = ro->topk_ids;
    c.wts_user = ro->topk_weights;
    c.logits_user = ro->logits;
    c.counts_user = ro->counts;
    c.offsets_user = ro->offsets;
    c.perm_user = ro->perm;
    c.invperm_user = ro->inv_perm;
  }
  c.ws = ws;
  c.ws_bytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
  c.stream = stream;
  c.phases = PH_ROUTE | PH_PERMUTE | PH_FFN | PH_COMBINE;
  c.reset_err = 1;
  return launch(c);
}

moe_status moe_pack_weights(const moe_problem *p, const moe_weights *src, const moe_weights *dst,
                            hipStream_t stream) {
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  moe_problem q = *p;
  q.w_layout = MOE_W_ROWMAJOR;
  moe_status st = validate_problem(&q);
  if (st != MOE_OK) return st;
  if (!src || !dst) return MOE_ERR_INVALID_ARGUMENT;
  const size_t wsz = dtype_size(p->w_dtype);
  struct Job {
    const void *s;
    void *d;
    size_t nmat, rows, cols_bytes;
  } jobs[6] = {
      {src->w_gate, const_cast<void *>(dst->w_gate), (size_t)p->E, (size_t)p->n, (size_t)p->d * wsz},
      {src->w_up, const_cast<void *>(dst->w_up), (size_t)p->E, (size_t)p->n, (size_t)p->d * wsz},
      {src->w_down, const_cast<void *>(dst->w_down), (size_t)p->E, (size_t)p->d, (size_t)p->n * wsz},
      {src->sh_gate, const_cast<void *>(dst->sh_gate), 1, (size_t)p->n, (size_t)p->d * wsz},
      {src->sh_up, const_cast<void *>(dst->sh_up), 1, (size_t)p->n, (size_t)p->d * wsz},
      {src->sh_down, const_cast<void *>(dst->sh_down), 1, (size_t)p->d, (size_t)p->n * wsz},
  };
  const int njobs = p->n_shared ? 6 : 3;
  for (int i = 0; i < njobs; ++i) {
    const Job &J = jobs[i];
    if (!J.s || !J.d || !aligned16(J.s) || !aligned16(J.d)) return MOE_ERR_INVALID_ARGUMENT;
    const size_t bytes = J.nmat * J.rows * J.cols_bytes;
    const uintptr_t a = reinterpret_cast<uintptr_t>(J.s), b = reinterpret_cast<uintptr_t>(J.d);
    if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARGUMENT;  // overlap
  }
  for (int i = 0; i < njobs; ++i) {
    const Job &J = jobs[i];
    const size_t nchunks = J.nmat * J.rows * J.cols_bytes / 16;
    size_t blocks = (nchunks + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const uint4 *>(J.s),
                       static_cast<uint4 *>(J.d), nchunks, (int)(J.cols_bytes / 16));
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

moe_status moe_last_device_error(const void *ws, hipStream_t stream) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  int magic = 0, err = 0;
  const int *c = static_cast<const int *>(ws);
  if (hipMemcpy(&magic, c + kSlotInts * C_MAGIC, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  if (hipMemcpy(&err, c + kSlotInts * C_ERR, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  if (magic != kMagic || err != 0) return MOE_ERR_DEVICE_FAULT;
  return MOE_OK;
}

}  // extern "C"
