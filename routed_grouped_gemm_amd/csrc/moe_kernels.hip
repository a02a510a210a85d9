// moe_kernels.hip -- the MoE-layer forward for gfx950 (MI355X), behind the C ABI of moe.h.
//
// One persistent kernel runs the whole layer.  Its work items are pulled from an atomic
// ticket counter in the workspace (the global task queue with an atomic counter of the
// Weave review, section 2.2; the work-conserving tile scheduler of the FlashMoE
// explainer, section 四), in this order:
//
//   Z  clear the per-m-tile dependency counters
//   L  router logits: 16 tokens x 64 experts per item (MFMA)
//   K  top-k + softmax over the kept logits for a chunk of tokens, and the chunk's
//      per-expert histogram; the last K item to finish builds the plan (scan of the
//      histograms, expert offsets, m-tile offsets)
//   SG shared-expert gate/up items (need no routing, so they overlap the plan)
//   S  stable scatter of a chunk: perm / inv_perm
//   G  gate/up items (expert, m-tile, 64 H columns): gathered token rows x W_gate/W_up,
//      SwiGLU in registers, H written once
//   D  down items (m-tile, 128 output columns): H rows x W_down -> Y
//   C  combine items: out[t] = sum_j w[t,j] * Y[inv_perm[t*k+j]] (+ Y_shared[t]), fixed
//      slot order, float32, one rounding, no float atomics
//
// A work item only ever waits for items with smaller tickets.  Those were taken by
// workgroups that are running, so every wait ends whatever the grid size or how many
// workgroups are resident.  Every wait is also bounded in time; a timeout sets a fault
// flag that makes every later wait give up, so the kernel always exits.
//
// Expert tiles: weights are the MFMA A operand (rows = output channels, K contiguous, one
// 16-byte load per lane straight from HBM into registers, double-buffered), token rows
// are the B operand (gathered rows staged through LDS with an XOR swizzle).  This is the
// operand-swapped form that suits small M (GC-MoE article, "two MMA implementations"):
// the weight stream, the HBM-bound part, is read exactly once per item and never
// passes through LDS.
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

enum : int { WF32 = 0, WBF16 = 1, WFP8 = 2 };

// K elements per 16-byte lane load (KU), loads per chunk (FL), chunk (KC = FL*KU):
// every chunk stages 512 bytes of each activation row.
template <int WT> struct WTr;
template <> struct WTr<WF32> { static constexpr int FL = 8, KU = 16, KC = 128, WSZ = 4, ASZ = 4; };
template <> struct WTr<WBF16> { static constexpr int FL = 8, KU = 32, KC = 256, WSZ = 2, ASZ = 2; };
template <> struct WTr<WFP8> { static constexpr int FL = 4, KU = 64, KC = 256, WSZ = 1, ASZ = 2; };
constexpr int kRowChunkBytes = 512;

struct KParams {
  int T, d, n, E, k, S;
  int phases;
  int bm, tk;
  int n_lt, n_le, n_kc, n_shmt, nt_gu, nt_dn, n_comb, n_zero, mt_cap;
  int n_static;  // Z + L + K + SG + S tickets
  int schedule;  // 0 dynamic, 1 static
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
  void *H, *Y;
};

// ---------------------------------------------------------------------------------
// scoped atomics and bounded waits
// ---------------------------------------------------------------------------------
__device__ __forceinline__ int ld_acquire(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_relaxed(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_acq_rel(int *p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr uint64_t kSpinTicks = 200000000ull;  // ~2 s of the 100 MHz wall clock

// Thread 0 only: wait until *p >= target.  False on timeout or an earlier fault.
__device__ bool spin_geq(const int *p, int target, int *err) {
  if (ld_acquire(p) >= target) return true;
  const uint64_t t0 = wall_clock64();
  for (;;) {
    __builtin_amdgcn_s_sleep(2);
    if (ld_acquire(p) >= target) return true;
    if (ld_relaxed(err) != 0) return false;
    if (wall_clock64() - t0 > kSpinTicks) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
}

// ---------------------------------------------------------------------------------
// shared memory
// ---------------------------------------------------------------------------------
template <int MG> struct Smem {
  union {
    struct {
      char act[2][MG * 16 * kRowChunkBytes];
    } g;
    struct {
      int ids[256];
      float wl[kWaves][kMaxK];
      int hist[kMaxE];
      int tmp[kMaxE];
    } r;
  } u;
  int rows[MG * 16];
  int bcast[4];
};

// ---------------------------------------------------------------------------------
// numeric helpers
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  // exact for values with <= 8 significant bits (fp8 values)
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// 8 OCP e4m3 codes -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t a, uint32_t b) {
  f2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, false);
  f2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)a, true);
  f2v p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
  f2v p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, true);
  uint4 r;
  r.x = pack_hi16(p0.x, p0.y);
  r.y = pack_hi16(p1.x, p1.y);
  r.z = pack_hi16(p2.x, p2.y);
  r.w = pack_hi16(p3.x, p3.y);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// monotone map float -> uint32 (after -0.0 -> +0.0), larger float -> larger key
__device__ __forceinline__ uint32_t ordered_key(float v) {
  v = v + 0.0f;  // -0.0 + 0.0 = +0.0 under round-to-nearest
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k ^ 0x80000000u) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------------
// MFMA tile core: acc[NF][MG] (+)= W[NF frags of 16 rows, K] . A[MG groups of 16 rows, K]^T
//
// lane l = 16*g + j: holds weight row (frag base + j), K bytes [64*f + 16*g, +16) of
// every 64-byte step f; the activation operand of token (mg*16 + j) over the same K
// positions; result D[4*g + r][j] = channel (frag base + 4*g + r), token (mg*16 + j).
// ---------------------------------------------------------------------------------
template <int WT, int NF, int MG> struct Gemm {
  using Tr = WTr<WT>;
  static constexpr int FL = Tr::FL;
  static constexpr int BMR = MG * 16;
  static constexpr int STG = BMR * (kRowChunkBytes / 16) / kThreads;  // uint4 per thread

  // wrow[f]: this lane's weight row start (+16*g already added); sc[f]: fp8 scale row of
  // the frag's 128-row block (nullptr otherwise); arow: activation matrix, `rows` LDS
  // list of its row indices (valid, clamped); kbytes_a: bytes per activation row.
  __device__ static void run(f4 (&acc)[NF][MG], const char *const (&wrow)[NF],
                             const float *const (&sc)[NF], const char *arow, size_t kbytes_a,
                             const int *rows, char (*act)[BMR * kRowChunkBytes], int K, int ngroups) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, j = lane & 15;
    const int nch = K / Tr::KC;
#pragma unroll
    for (int a = 0; a < NF; ++a)
#pragma unroll
      for (int b = 0; b < MG; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

    uint4 wA[NF][FL], wB[NF][FL];
    uint4 st[STG];
    const int nk128 = K / 128;

    auto load_w = [&](uint4(&W)[NF][FL], int c) {
#pragma unroll
      for (int f = 0; f < FL; ++f)
#pragma unroll
        for (int a = 0; a < NF; ++a)
          W[a][f] = *reinterpret_cast<const uint4 *>(wrow[a] + (size_t)c * (FL * 64) + f * 64);
    };
    auto load_a = [&](int c) {
#pragma unroll
      for (int s = 0; s < STG; ++s) {
        const int idx = tid + kThreads * s;
        const int r = idx >> 5, col = idx & 31;
        st[s] = *reinterpret_cast<const uint4 *>(arow + (size_t)rows[r] * kbytes_a +
                                                 (size_t)c * kRowChunkBytes + col * 16);
      }
    };
    auto store_a = [&](int buf) {
#pragma unroll
      for (int s = 0; s < STG; ++s) {
        const int idx = tid + kThreads * s;
        const int r = idx >> 5, col = idx & 31;
        *reinterpret_cast<uint4 *>(act[buf] + r * kRowChunkBytes + ((col ^ (r & 31)) << 4)) = st[s];
      }
    };
    auto compute = [&](const uint4(&W)[NF][FL], int buf, int c) {
      const char *A = act[buf];
      if constexpr (WT == WFP8) {
        float s0[NF], s1[NF];
#pragma unroll
        for (int a = 0; a < NF; ++a) {
          s0[a] = sc[a][2 * c];
          s1[a] = (2 * c + 1 < nk128) ? sc[a][2 * c + 1] : 0.f;
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          f4 tmp[NF][MG];
#pragma unroll
          for (int a = 0; a < NF; ++a)
#pragma unroll
            for (int b = 0; b < MG; ++b) tmp[a][b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ff = 0; ff < 2; ++ff) {
            const int f = blk * 2 + ff;
#pragma unroll
            for (int b = 0; b < MG; ++b) {
              if (b < ngroups) {
                const int r = b * 16 + j;
                const int c0 = f * 8 + 2 * g;
                const uint4 a0 = *reinterpret_cast<const uint4 *>(A + r * kRowChunkBytes + ((c0 ^ (r & 31)) << 4));
                const uint4 a1 = *reinterpret_cast<const uint4 *>(A + r * kRowChunkBytes + (((c0 + 1) ^ (r & 31)) << 4));
                const bf16x8 b0 = __builtin_bit_cast(bf16x8, a0);
                const bf16x8 b1 = __builtin_bit_cast(bf16x8, a1);
#pragma unroll
                for (int a = 0; a < NF; ++a) {
                  const uint4 w = W[a][f];
                  tmp[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w.x, w.y), b0, tmp[a][b], 0, 0, 0);
                  tmp[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(w.z, w.w), b1, tmp[a][b], 0, 0, 0);
                }
              }
            }
          }
#pragma unroll
          for (int a = 0; a < NF; ++a) {
            const float s = blk == 0 ? s0[a] : s1[a];
#pragma unroll
            for (int b = 0; b < MG; ++b) acc[a][b] += tmp[a][b] * s;
          }
        }
      } else {
#pragma unroll
        for (int f = 0; f < FL; ++f) {
#pragma unroll
          for (int b = 0; b < MG; ++b) {
            if (b < ngroups) {
              const int r = b * 16 + j;
              const int c0 = f * 4 + g;
              const uint4 av = *reinterpret_cast<const uint4 *>(A + r * kRowChunkBytes + ((c0 ^ (r & 31)) << 4));
#pragma unroll
              for (int a = 0; a < NF; ++a) {
                const uint4 w = W[a][f];
                if constexpr (WT == WBF16) {
                  acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      __builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, av), acc[a][b], 0, 0, 0);
                } else {
                  acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), __uint_as_float(av.x), acc[a][b], 0, 0, 0);
                  acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), __uint_as_float(av.y), acc[a][b], 0, 0, 0);
                  acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), __uint_as_float(av.z), acc[a][b], 0, 0, 0);
                  acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), __uint_as_float(av.w), acc[a][b], 0, 0, 0);
                }
              }
            }
          }
        }
      }
    };

    load_w(wA, 0);
    load_a(0);
    store_a(0);
    for (int c = 0; c < nch; c += 2) {
      const bool h1 = c + 1 < nch;
      if (h1) {
        load_w(wB, c + 1);
        load_a(c + 1);
      }
      __syncthreads();
      compute(wA, 0, c);
      if (!h1) break;
      store_a(1);
      const bool h2 = c + 2 < nch;
      if (h2) {
        load_w(wA, c + 2);
        load_a(c + 2);
      }
      __syncthreads();
      compute(wB, 1, c + 1);
      if (h2) store_a(0);
    }
  }
};

// ---------------------------------------------------------------------------------
// workgroup-level sync helpers
// ---------------------------------------------------------------------------------
// Every thread: make this workgroup's global writes visible at agent scope, then bump
// `counter` once.  Returns the counter's old value (valid in thread 0 only).
__device__ __forceinline__ int wg_signal(int *counter) {
  __threadfence();
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return old;
}

template <int MG>
__device__ __forceinline__ bool wg_wait(const int *p, int target, int *err, Smem<MG> &sm) {
  __syncthreads();
  if (threadIdx.x == 0) sm.bcast[1] = spin_geq(p, target, err) ? 1 : 0;
  __syncthreads();
  const bool ok = sm.bcast[1] != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return ok;
}

// ---------------------------------------------------------------------------------
// phase items
// ---------------------------------------------------------------------------------
template <int MG>
__device__ void zero_item(const KParams &P, int i) {
  const int lo = i * kZeroPerItem;
  for (int q = threadIdx.x; q < kZeroPerItem; q += kThreads) {
    const int idx = lo + q;
    if (idx < P.mt_cap) P.gudone[idx] = 0;
  }
}

// router logits for 16 tokens x 64 experts
template <int WT, int MG>
__device__ void logits_item(const KParams &P, int i, Smem<MG> &sm) {
  constexpr int RT = (WT == WF32) ? WF32 : WBF16;  // the router runs in the activation dtype
  using G = Gemm<RT, 1, 1>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int lt = i / P.n_le, le = i % P.n_le;
  const int t0 = lt * kLogitTokens, e0 = le * kLogitExperts;
  const int ntok = min(kLogitTokens, P.T - t0);
  if (tid < 16) sm.rows[tid] = t0 + min(tid, ntok - 1);
  __syncthreads();
  const size_t asz = WTr<RT>::ASZ;
  const int er = min(e0 + wave * 16 + j, P.E - 1);
  const char *wrow[1] = {reinterpret_cast<const char *>(P.wr) + (size_t)er * P.d * asz + g * 16};
  const float *sc[1] = {nullptr};
  f4 acc[1][1];
  G::run(acc, wrow, sc, reinterpret_cast<const char *>(P.x), (size_t)P.d * asz, sm.rows,
         reinterpret_cast<char(*)[16 * kRowChunkBytes]>(sm.u.g.act), P.d, 1);
  if (j < ntok) {
    const int t = t0 + j;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = e0 + wave * 16 + 4 * g + r;
      if (e < P.E) P.logits[(size_t)t * P.E + e] = acc[0][0][r] + (P.bias ? P.bias[e] : 0.f);
    }
  }
}

// wave-level exclusive scan of in[0..N) -> out[0..N+1) (out[N] = total); one wave runs it
__device__ void wave_excl_scan(const int *in, int *out, int N, int lane) {
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

// The plan: per-expert scan of the chunk histograms (chunk bases, in place), counts,
// offsets, m-tile offsets.  One workgroup.
template <int MG>
__device__ void plan_wg(const KParams &P, Smem<MG> &sm) {
  const int tid = threadIdx.x, E = P.E, nkc = P.n_kc;
  int *cnt = sm.u.r.hist;
  int *mtc = sm.u.r.tmp;
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
    for (int c0 = 0; c0 < nkc; c0 += 16) {
      int h[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) h[q] = (c0 + q < nkc) ? P.hist[(size_t)(c0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (c0 + q < nkc) P.hist[(size_t)(c0 + q) * E + e] = run;
        run += h[q];
      }
    }
    cnt[e] = run;
    mtc[e] = (run + P.bm - 1) / P.bm;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  if (wave == 0) wave_excl_scan(cnt, P.offsets, E, lane);
  if (wave == 1) wave_excl_scan(mtc, P.mtoff, E, lane);
  for (int e = tid; e < E; e += kThreads) P.counts[e] = cnt[e];
  __syncthreads();
  if (tid == 0) P.ctrl[C_NMT] = P.mtoff[E];
  wg_signal(P.ctrl + C_PLAN);
}

// top-k + softmax + chunk histogram for tokens [c*tk, min(T, (c+1)*tk))
template <int MG>
__device__ void topk_item(const KParams &P, int c, Smem<MG> &sm) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = c * P.tk, ntok = min(P.tk, P.T - t0), k = P.k, E = P.E;
  if (P.phases & PH_IDS_GIVEN) {
    for (int q = tid; q < ntok * k; q += kThreads) sm.u.r.ids[q] = P.ids[(size_t)t0 * k + q];
  } else {
    for (int tt = wave; tt < ntok; tt += kWaves) {
      const int t = t0 + tt;
      const float *Lr = P.logits + (size_t)t * E;
      uint64_t key[kMaxE / 64];
#pragma unroll
      for (int q = 0; q < kMaxE / 64; ++q) {
        const int e = q * 64 + lane;
        key[q] = (e < E) ? ((uint64_t)ordered_key(Lr[e]) << 32) | (uint32_t)(E - 1 - e) : 0ull;
      }
      for (int jj = 0; jj < k; ++jj) {
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < kMaxE / 64; ++q) best = key[q] > best ? key[q] : best;
        uint64_t m = best;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const uint64_t o = __shfl_xor(m, off, 64);
          m = o > m ? o : m;
        }
#pragma unroll
        for (int q = 0; q < kMaxE / 64; ++q)
          if (key[q] == m) key[q] = 0ull;
        if (lane == 0) {
          sm.u.r.ids[tt * k + jj] = E - 1 - (int)(uint32_t)(m & 0xffffffffu);
          sm.u.r.wl[wave][jj] = key_value((uint32_t)(m >> 32));
        }
      }
      // softmax over the kept logits, summed in slot order
      if (lane == 0) {
        const float l0 = sm.u.r.wl[wave][0];
        float s = 0.f;
        for (int jj = 0; jj < k; ++jj) {
          const float z = expf(sm.u.r.wl[wave][jj] - l0);
          sm.u.r.wl[wave][jj] = z;
          s += z;
        }
        for (int jj = 0; jj < k; ++jj) {
          P.wts[(size_t)t * k + jj] = sm.u.r.wl[wave][jj] / s;
          P.ids[(size_t)t * k + jj] = sm.u.r.ids[tt * k + jj];
        }
      }
    }
  }
  // histogram of the chunk (integer counts; order-independent)
  for (int e = tid; e < E; e += kThreads) sm.u.r.hist[e] = 0;
  __syncthreads();
  for (int q = tid; q < ntok * k; q += kThreads) {
    const int e = sm.u.r.ids[q];
    if (e >= 0 && e < E) atomicAdd(&sm.u.r.hist[e], 1);
    else __hip_atomic_store(P.ctrl + C_ERR, 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) P.hist[(size_t)c * E + e] = sm.u.r.hist[e];
  const int old = wg_signal(P.ctrl + C_KDONE);
  if (tid == 0) sm.bcast[2] = (old == P.n_kc - 1) ? 1 : 0;
  __syncthreads();
  if (sm.bcast[2] && (P.phases & PH_PERMUTE)) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    plan_wg(P, sm);
  }
}

// stable scatter of chunk c: position of slot (t, j) with expert e is
//   offsets[e] + (slots of e in earlier chunks) + (slots of e in earlier tokens of this chunk)
template <int MG>
__device__ void scatter_item(const KParams &P, int c, Smem<MG> &sm) {
  const int tid = threadIdx.x;
  const int t0 = c * P.tk, ntok = min(P.tk, P.T - t0), k = P.k, E = P.E;
  const int nq = ntok * k;
  for (int q = tid; q < nq; q += kThreads) sm.u.r.ids[q] = P.ids[(size_t)t0 * k + q];
  __syncthreads();
  for (int q = tid; q < nq; q += kThreads) {
    const int e = sm.u.r.ids[q];
    if (e < 0 || e >= E) continue;
    const int first = (q / k) * k;
    int rank = 0;
    for (int q2 = 0; q2 < first; ++q2) rank += (sm.u.r.ids[q2] == e) ? 1 : 0;
    const int p = P.offsets[e] + P.hist[(size_t)c * E + e] + rank;
    const int slot = t0 * k + q;
    P.perm[p] = slot;
    P.inv_perm[slot] = p;
  }
}

// which routed expert owns global m-tile g: the e with mtoff[e] <= g < mtoff[e+1]
__device__ __forceinline__ int find_expert(const int *mtoff, int E, int g) {
  int lo = 0, hi = E;  // upper_bound over mtoff[0..E]
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (mtoff[mid] <= g) lo = mid + 1;
    else hi = mid;
  }
  return lo - 1;
}

template <int WT> struct ActT { using type = uint16_t; };
template <> struct ActT<WF32> { using type = float; };

template <int WT>
__device__ __forceinline__ void store4(void *base, size_t idx, f4 v) {
  if constexpr (WT == WF32) {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 u;
    u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(base) + idx) = u;
  }
}

// gate/up item: rows (tokens) of one m-tile x 64 H columns; SwiGLU in registers
template <int WT, int MG>
__device__ void gateup_item(const KParams &P, bool shared, int i, Smem<MG> &sm) {
  using G = Gemm<WT, 2, MG>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, j = lane & 15;
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
    e = find_expert(P.mtoff, P.E, gm);
    const int mt = gm - P.mtoff[e];
    row0 = P.offsets[e] + mt * P.bm;
    m = min(P.bm, P.counts[e] - mt * P.bm);
    hrow0 = row0;
    counter = P.n_shmt + gm;
  }
  for (int r = tid; r < G::BMR; r += kThreads) {
    const int rr = min(r, m - 1);
    int tok = shared ? row0 + rr : P.perm[row0 + rr] / P.k;
    tok = min(max(tok, 0), P.T - 1);
    sm.rows[r] = tok;
  }
  __syncthreads();
  const size_t wsz = WTr<WT>::WSZ, asz = WTr<WT>::ASZ;
  const int n0 = nt * kGuCols + wave * 16;
  const char *wgb = reinterpret_cast<const char *>(shared ? P.shg : P.wg);
  const char *wub = reinterpret_cast<const char *>(shared ? P.shu : P.wu);
  const size_t emat = shared ? 0 : (size_t)e * P.n * P.d * wsz;
  const size_t rowoff = (size_t)(n0 + j) * P.d * wsz + g * 16;
  const char *wrow[2] = {wgb + emat + rowoff, wub + emat + rowoff};
  const float *sc[2] = {nullptr, nullptr};
  if constexpr (WT == WFP8) {
    const int nkb = P.d / 128;
    const size_t soff = (shared ? 0 : (size_t)e * (P.n / 128) * nkb) + (size_t)(n0 / 128) * nkb;
    sc[0] = (shared ? P.shsg : P.sg) + soff;
    sc[1] = (shared ? P.shsu : P.su) + soff;
  }
  f4 acc[2][MG];
  const int ngroups = (m + 15) >> 4;
  G::run(acc, wrow, sc, reinterpret_cast<const char *>(P.x), (size_t)P.d * asz, sm.rows,
         reinterpret_cast<char(*)[G::BMR * kRowChunkBytes]>(sm.u.g.act), P.d, ngroups);
#pragma unroll
  for (int b = 0; b < MG; ++b) {
    const int r = b * 16 + j;
    if (r < m) {
      f4 h;
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = silu_mul(acc[0][b][q], acc[1][b][q]);
      store4<WT>(P.H, (hrow0 + r) * (size_t)P.n + n0 + 4 * g, h);
    }
  }
  wg_signal(P.gudone + counter);
}

// down item: rows of one m-tile x 128 output columns
template <int WT, int MG>
__device__ bool down_item(const KParams &P, int i, Smem<MG> &sm) {
  using G = Gemm<WT, 2, MG>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int gm = i / P.nt_dn, dt = i % P.nt_dn;
  if (!wg_wait(P.gudone + gm, P.nt_gu, P.ctrl + C_ERR, sm)) return false;
  const bool shared = gm < P.n_shmt;
  int e, m;
  size_t row0;
  if (shared) {
    e = P.E;
    const int t0 = gm * P.bm;
    m = min(P.bm, P.T - t0);
    row0 = (size_t)P.T * P.k + t0;
  } else {
    const int gr = gm - P.n_shmt;
    e = find_expert(P.mtoff, P.E, gr);
    const int mt = gr - P.mtoff[e];
    row0 = (size_t)P.offsets[e] + mt * P.bm;
    m = min(P.bm, P.counts[e] - mt * P.bm);
  }
  for (int r = tid; r < G::BMR; r += kThreads) sm.rows[r] = (int)(row0 + min(r, m - 1));
  __syncthreads();
  const size_t wsz = WTr<WT>::WSZ, asz = WTr<WT>::ASZ;
  const int d0 = dt * kDnCols + wave * 32;
  const char *wdb = reinterpret_cast<const char *>(shared ? P.shd : P.wd);
  const size_t emat = shared ? 0 : (size_t)e * P.d * P.n * wsz;
  const int r0 = min(d0 + j, P.d - 1), r1 = min(d0 + 16 + j, P.d - 1);
  const char *wrow[2] = {wdb + emat + (size_t)r0 * P.n * wsz + g * 16,
                         wdb + emat + (size_t)r1 * P.n * wsz + g * 16};
  const float *sc[2] = {nullptr, nullptr};
  if constexpr (WT == WFP8) {
    const int nkb = P.n / 128;
    const float *sb = (shared ? P.shsd : P.sd) + (shared ? 0 : (size_t)e * (P.d / 128) * nkb);
    sc[0] = sb + (size_t)(min(d0, P.d - 1) / 128) * nkb;
    sc[1] = sb + (size_t)(min(d0 + 16, P.d - 1) / 128) * nkb;
  }
  f4 acc[2][MG];
  const int ngroups = (m + 15) >> 4;
  G::run(acc, wrow, sc, reinterpret_cast<const char *>(P.H), (size_t)P.n * asz, sm.rows,
         reinterpret_cast<char(*)[G::BMR * kRowChunkBytes]>(sm.u.g.act), P.n, ngroups);
#pragma unroll
  for (int b = 0; b < MG; ++b) {
    const int r = b * 16 + j;
    if (r < m) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c = d0 + 16 * a + 4 * g;
        if (c < P.d) store4<WT>(P.Y, (row0 + r) * (size_t)P.d + c, acc[a][b]);
      }
    }
  }
  wg_signal(P.ctrl + C_DDONE);
  return true;
}

// combine: out[t] = sum_j w[t,j] * Y[inv_perm[t*k+j]] (+ Y[T*k + t]), float32, slot order
template <int WT, int MG>
__device__ void combine_item(const KParams &P, int c, Smem<MG> &sm) {
  using A = typename ActT<WT>::type;
  constexpr int VEC = 16 / sizeof(A);
  const int t0 = c * kCombineTokens, ntok = min(kCombineTokens, P.T - t0);
  const int nv = P.d / VEC;
  const A *Y = reinterpret_cast<const A *>(P.Y);
  A *out = reinterpret_cast<A *>(P.out);
  for (int q = threadIdx.x; q < ntok * nv; q += kThreads) {
    const int t = t0 + q / nv, v = q % nv;
    float acc[VEC];
#pragma unroll
    for (int z = 0; z < VEC; ++z) acc[z] = 0.f;
    for (int jj = 0; jj < P.k; ++jj) {
      const float w = P.wts[(size_t)t * P.k + jj];
      const int p = P.inv_perm[(size_t)t * P.k + jj];
      const uint4 raw = *reinterpret_cast<const uint4 *>(Y + (size_t)p * P.d + v * VEC);
      if constexpr (WT == WF32) {
        const float *f = reinterpret_cast<const float *>(&raw);
#pragma unroll
        for (int z = 0; z < VEC; ++z) acc[z] += w * f[z];
      } else {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(&raw);
#pragma unroll
        for (int z = 0; z < VEC; ++z) acc[z] += w * bf2f(h[z]);
      }
    }
    if (P.S) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(Y + ((size_t)P.T * P.k + t) * P.d + v * VEC);
      if constexpr (WT == WF32) {
        const float *f = reinterpret_cast<const float *>(&raw);
#pragma unroll
        for (int z = 0; z < VEC; ++z) acc[z] += f[z];
      } else {
        const uint16_t *h = reinterpret_cast<const uint16_t *>(&raw);
#pragma unroll
        for (int z = 0; z < VEC; ++z) acc[z] += bf2f(h[z]);
      }
    }
    uint4 o;
    if constexpr (WT == WF32) {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3]));
    } else {
      uint32_t wv[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) wv[z] = (uint32_t)f2bf(acc[2 * z]) | ((uint32_t)f2bf(acc[2 * z + 1]) << 16);
      o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    *reinterpret_cast<uint4 *>(out + (size_t)t * P.d + v * VEC) = o;
  }
}

// ---------------------------------------------------------------------------------
// the persistent kernel
// ---------------------------------------------------------------------------------
template <int WT, int MG>
__global__ __launch_bounds__(kThreads) void moe_persistent(KParams P) {
  __shared__ Smem<MG> sm;
  const int tid = threadIdx.x;
  int *ctrl = P.ctrl;
  int *err = ctrl + C_ERR;
  if (ld_relaxed(ctrl + C_MAGIC) != kMagic) {
    if (tid == 0) __hip_atomic_store(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int n_Z = (P.phases & PH_FFN) ? P.n_zero : 0;
  const int n_L = (P.phases & PH_ROUTE) ? P.n_lt * P.n_le : 0;
  const int n_K = (P.phases & (PH_ROUTE | PH_PERMUTE)) ? P.n_kc : 0;
  const int n_SG = (P.phases & PH_FFN) ? P.n_shmt * P.nt_gu : 0;
  const int n_S = (P.phases & PH_PERMUTE) ? P.n_kc : 0;
  const bool dyn = (P.phases & (PH_FFN | PH_COMBINE)) != 0;
  bool zero_seen = false, logits_seen = false, plan_seen = false, scat_seen = false, dn_seen = false;
  int n_mt = 0;
  int step = 0;
  for (;;) {
    __syncthreads();
    if (P.schedule == 0) {
      if (tid == 0) sm.bcast[0] = __hip_atomic_fetch_add(ctrl + C_TICKET, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
    }
    int i = P.schedule == 0 ? sm.bcast[0] : (int)blockIdx.x + step * (int)gridDim.x;
    ++step;
    if (i < n_Z) {
      zero_item<MG>(P, i);
      wg_signal(ctrl + C_ZDONE);
      continue;
    }
    i -= n_Z;
    if (i < n_L) {
      logits_item<WT, MG>(P, i, sm);
      wg_signal(ctrl + C_LDONE);
      continue;
    }
    i -= n_L;
    if (i < n_K) {
      if (!(P.phases & PH_IDS_GIVEN) && !logits_seen) {
        if (!wg_wait(ctrl + C_LDONE, n_L, err, sm)) break;
        logits_seen = true;
      }
      topk_item<MG>(P, i, sm);
      continue;
    }
    i -= n_K;
    if (i < n_SG) {
      if (!zero_seen) {
        if (!wg_wait(ctrl + C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      gateup_item<WT, MG>(P, true, i, sm);
      continue;
    }
    i -= n_SG;
    if (i < n_S) {
      if (!plan_seen) {
        if (!wg_wait(ctrl + C_PLAN, 1, err, sm)) break;
        plan_seen = true;
      }
      scatter_item<MG>(P, i, sm);
      wg_signal(ctrl + C_SDONE);
      continue;
    }
    i -= n_S;
    if (!dyn) break;
    if (!plan_seen) {
      if (!wg_wait(ctrl + C_PLAN, 1, err, sm)) break;
      plan_seen = true;
    }
    if (n_mt == 0) n_mt = ld_relaxed(ctrl + C_NMT);
    const int n_G = n_mt * P.nt_gu;
    if (i < n_G) {
      if (!scat_seen) {
        if (!wg_wait(ctrl + C_SDONE, n_S, err, sm)) break;
        scat_seen = true;
      }
      if (!zero_seen) {
        if (!wg_wait(ctrl + C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      gateup_item<WT, MG>(P, false, i, sm);
      continue;
    }
    i -= n_G;
    const int n_D = (n_mt + P.n_shmt) * P.nt_dn;
    if (i < n_D) {
      if (!zero_seen) {  // the dependency counters must be cleared before they are read
        if (!wg_wait(ctrl + C_ZDONE, n_Z, err, sm)) break;
        zero_seen = true;
      }
      if (!down_item<WT, MG>(P, i, sm)) break;
      continue;
    }
    i -= n_D;
    if (i < P.n_comb) {
      if (!dn_seen) {
        if (!wg_wait(ctrl + C_DDONE, n_D, err, sm)) break;
        dn_seen = true;
      }
      combine_item<WT, MG>(P, i, sm);
      continue;
    }
    break;
  }
  // the last workgroup out resets the control block for the next call
  __syncthreads();
  if (tid == 0) {
    const int old = add_acq_rel(ctrl + C_EXIT, 1);
    if (old == (int)gridDim.x - 1) {
      for (int s = C_TICKET; s <= C_NMT; ++s) ctrl[s] = 0;
      __threadfence();
    }
  }
}

__global__ void ws_init_kernel(int *ctrl, size_t nwords) {
  for (size_t q = blockIdx.x * (size_t)blockDim.x + threadIdx.x; q < nwords; q += (size_t)gridDim.x * blockDim.x)
    ctrl[q] = (q == C_MAGIC) ? kMagic : 0;
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------
typedef void (*KernelFn)(KParams);

template <int WT> KernelFn pick_kernel(int mg) {
  switch (mg) {
    case 1: return moe_persistent<WT, 1>;
    case 2: return moe_persistent<WT, 2>;
    case 4: return moe_persistent<WT, 4>;
    default: return moe_persistent<WT, 8>;
  }
}

KernelFn kernel_for(int w_dtype, int mg) {
  if (w_dtype == MOE_F32) return pick_kernel<WF32>(mg);
  if (w_dtype == MOE_BF16) return pick_kernel<WBF16>(mg);
  return pick_kernel<WFP8>(mg);
}

struct DevInfo {
  int cus = 0;
  int occ[3][4] = {};
};

std::mutex g_mu;
DevInfo g_dev[64];
bool g_have[64];

moe_status device_info(int dev, int w_dtype, int mg, int *cus, int *occ) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (dev < 0 || dev >= 64) return MOE_ERR_HIP;
  DevInfo &D = g_dev[dev];
  if (!g_have[dev]) {
    if (hipDeviceGetAttribute(&D.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
    g_have[dev] = true;
  }
  const int mi = mg == 1 ? 0 : mg == 2 ? 1 : mg == 4 ? 2 : 3;
  int &o = D.occ[w_dtype][mi];
  if (o == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(kernel_for(w_dtype, mg)),
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
  const moe_route_out *ro;
  int32_t *ids_user;
  float *wts_user, *logits_user;
  const int32_t *ids_in;
  int32_t *counts_user, *offsets_user, *perm_user, *invperm_user;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
  int phases;
  const moe_launch_options *opts;
};

moe_status launch(const Call &c) {
  const moe_problem *p = c.p;
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (!c.ws || (reinterpret_cast<uintptr_t>(c.ws) & 255u)) return MOE_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(p);
  if (c.ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (c.opts && (c.opts->grid_wgs < 0 || c.opts->schedule < 0 || c.opts->schedule > 1))
    return c.opts && c.opts->schedule == 2 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARGUMENT;
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
  P.n_lt = L.n_lt;
  P.n_le = L.n_le;
  P.n_kc = L.n_kc;
  P.n_shmt = L.n_shmt;
  P.nt_gu = L.nt_gu;
  P.nt_dn = L.nt_dn;
  P.n_comb = L.n_comb;
  P.n_zero = L.n_zero;
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
  P.ids = c.ids_user ? c.ids_user : (c.ids_in ? const_cast<int *>(c.ids_in) : reinterpret_cast<int *>(ws + L.off_ids));
  P.wts = c.wts_user ? c.wts_user : reinterpret_cast<float *>(ws + L.off_wts);
  P.counts = c.counts_user ? c.counts_user : reinterpret_cast<int *>(ws + L.off_counts);
  P.offsets = c.offsets_user ? c.offsets_user : reinterpret_cast<int *>(ws + L.off_offsets);
  P.perm = c.perm_user ? c.perm_user : reinterpret_cast<int *>(ws + L.off_perm);
  P.inv_perm = c.invperm_user ? c.invperm_user : reinterpret_cast<int *>(ws + L.off_invperm);
  P.ctrl = reinterpret_cast<int *>(ws);
  P.gudone = reinterpret_cast<int *>(ws + L.off_gudone);
  P.hist = reinterpret_cast<int *>(ws + L.off_hist);
  P.mtoff = reinterpret_cast<int *>(ws + L.off_mtoff);
  P.H = ws + L.off_h;
  P.Y = ws + L.off_y;

  int n_items = 0;
  {
    const int n_Z = (P.phases & PH_FFN) ? P.n_zero : 0;
    const int n_L = (P.phases & PH_ROUTE) ? P.n_lt * P.n_le : 0;
    const int n_K = (P.phases & (PH_ROUTE | PH_PERMUTE)) ? P.n_kc : 0;
    const int n_SG = (P.phases & PH_FFN) ? P.n_shmt * P.nt_gu : 0;
    const int n_S = (P.phases & PH_PERMUTE) ? P.n_kc : 0;
    P.n_static = n_Z + n_L + n_K + n_SG + n_S;
    n_items = P.n_static;
    if (P.phases & PH_FFN)
      n_items += L.mt_routed_max * (P.nt_gu + P.nt_dn) + P.n_shmt * P.nt_dn + P.n_comb;
  }

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  int cus = 0, occ = 0;
  st = device_info(dev, p->w_dtype, L.tiles.mg, &cus, &occ);
  if (st != MOE_OK) return st;
  int grid = cus * occ;
  if (c.opts && c.opts->grid_wgs > 0) grid = c.opts->grid_wgs;
  P.schedule = c.opts ? c.opts->schedule : 0;
  if (P.schedule == 1 && grid > cus * occ) grid = cus * occ;  // static binding needs co-residency
  if (grid > n_items && P.schedule == 0) grid = n_items > 0 ? n_items : 1;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel_for(p->w_dtype, L.tiles.mg), dim3(grid), dim3(kThreads), 0, c.stream, P);
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

moe_status moe_last_device_error(const void *ws, hipStream_t stream) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  int ctrl[C_NSLOTS];
  if (hipMemcpy(ctrl, ws, sizeof(ctrl), hipMemcpyDeviceToHost) != hipSuccess) return MOE_ERR_HIP;
  if (ctrl[C_MAGIC] != kMagic || ctrl[C_ERR] != 0) return MOE_ERR_DEVICE_FAULT;
  return MOE_OK;
}

}  // extern "C"
