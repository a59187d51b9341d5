// gfx950 kernels for the AdaFlash verify + on-policy-distillation pass.
//
// What is computed is defined in include/av.h (after the Pith review page of
// "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion
// Drafters": "What carries the argument", Referee Report major comment 2 and
// minor comment 2, the free-parameter ledger).  This file is about how.
//
// fused_kernel -- the whole forward (+ gradient) pass in one launch.
//   One 1024-thread workgroup per CU, persistent, takes whole rows from an
//   atomic counter, longest first: in the dense layout every verified row is
//   handed out before any unverified one (they only need the argmax and a
//   zero gradient), so the last rows of the launch are the short ones.
//   Sweep 1 streams a row's zp and zq from HBM once and keeps as much of it
//   as fits on chip (per thread NR vectors in registers and NL in LDS, filled
//   by direct-to-LDS loads: about 70% of a 151936-wide bf16 row) while
//   folding every entry into online statistics:
//     max / sum exp / first argmax of zp (and zq there), max / sum exp of zq,
//     and K = sum exp(zq - m_q)(zq - zp), which gives the unclipped reverse KL.
//   The clip interval is entry-wise, so S (the softmax-gradient correction)
//   and the clipped-KL sum differ from their unclipped values only through
//   entries with |q_j log(q_j/p_j)| > tau.  A per-thread bound on q_j |ell_j|
//   (kept as running maxima of exp(zq_j - m) |zq_j - zp_j| and of zq_j)
//   certifies most regions clip-free; only regions that fail it are evaluated
//   entry by entry (on chip, or re-read).  Sweep 2 writes the fp32 gradient,
//   re-reading only the streamed part of the row.  HBM traffic per verified
//   bf16 entry: 4 bytes read, 4 written, plus ~1.2 bytes of re-read for the
//   part that did not fit on chip.
//
//   Rows never wait on each other.  A completed verified row publishes its
//   argmax and loss and counts itself on its request's arrival counter; the
//   workgroup whose count completes the request computes the accepted length
//   and the request loss, and the workgroup that leaves the kernel last sums
//   the request losses.  Every shared word is {tag, 32-bit payload} written
//   and read with agent-scope atomics (coherent across XCDs on its own, no
//   cache-wide fence); the tag is the launch epoch kept in the workspace, so
//   stale words of earlier launches never match and graph replays see a
//   fresh epoch.  A reader polls until the tag shows (bounded; on expiry the
//   launch reports AV_DEV_TIMEOUT).
//
// bwd_kernel -- gradient only, from saved row statistics; one streaming
//   sweep, the same float32 entry math as the fused pass (bit-identical).
// head_kernel -- length head: float64 dot product, sigmoid, rounding, clamp.

#include <limits.h>
#include <math.h>

#include "av.h"
#include "av_internal.h"

namespace avk {
namespace {

constexpr int kWaves = kBlock / 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// wide stores
//
// A store of more than 8 bytes keeps reading its data registers for a couple
// of cycles after it issues: on gfx950 a write to those registers one wait
// state later (and, with a register scalar offset, right after the store)
// can change what is stored.  The compiler's hazard handling assumes less, so
// every such store here is followed by an empty-bodied wait that keeps its
// data registers live across two wait states.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void settle16(const u32x4& v) { asm volatile("s_nop 1" ::"v"(v)); }
__device__ __forceinline__ void settle16(const f32x4& v) { asm volatile("s_nop 1" ::"v"(v)); }

__device__ __forceinline__ void store16(float* p, const f32x4& v) {
  *(f32x4*)p = v;
  settle16(v);
}
__device__ __forceinline__ void store16_nt(float* p, const f32x4& v) {
  __builtin_nontemporal_store(v, (f32x4*)p);
  settle16(v);
}
template <int AUX>
__device__ __forceinline__ void bstore16(const u32x4& v, __amdgpu_buffer_rsrc_t g, uint32_t voff,
                                         uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, g, voff, soff, AUX);
  settle16(v);
}

// ---------------------------------------------------------------------------
// tagged words and launch status
// ---------------------------------------------------------------------------

__device__ __forceinline__ void tput(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)v, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tget(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_ok(uint64_t w, uint32_t tag) {
  return (uint32_t)(w >> 32) == tag;
}
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Status bits live in the high halves of the dispenser word ctl[0] (so every
// later claim sees them) and of the exit word ctl[2] (so the workgroup that
// leaves last sees them).
__device__ __forceinline__ void raise_status(uint64_t* ctl, uint32_t bits) {
  const uint64_t v = (uint64_t)bits << 32;
  __hip_atomic_fetch_or(ctl, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_or(ctl + 2, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait: sleeps between polls (backing off up to ~0.4 us), and every
// few polls gives up if the launch already failed or the wall-clock bound is
// exceeded.  `ctl` is the launch's control block.
struct Waiter {
  long long t0, limit;
  uint64_t* ctl;
  int it;
  __device__ Waiter(uint64_t* c, long long lim) : t0(wall_clock64()), limit(lim), ctl(c), it(0) {}
  __device__ bool keep_going() {
    ++it;
    if ((it & 7) == 0) {
      if ((uint32_t)(tget(ctl + 2) >> 32) != 0u) return false;
      if (wall_clock64() - t0 > limit) {
        raise_status(ctl, AV_DEV_TIMEOUT);
        return false;
      }
    }
    const int n = it < 8 ? it : 8;
    for (int j = 0; j < n; ++j) __builtin_amdgcn_s_sleep(2);
    return true;
  }
};

// A wave-uniform value passed through an empty asm statement: values derived
// from it are recomputed where they are used instead of being hoisted out of
// the row loop (where they would hold scalar registers for the whole kernel).
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}
__device__ __forceinline__ float opaque_s(float x) {
  asm volatile("" : "+s"(x));
  return x;
}

// ---------------------------------------------------------------------------
// wave64 reductions (xor butterflies: every lane ends with the same bits);
// the fused row kernel uses the DPP row reductions further down
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wsumd(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// (value desc, index asc): the first index of the largest value.
__device__ __forceinline__ void amax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

// ---------------------------------------------------------------------------
// element access per variant
// ---------------------------------------------------------------------------

// Buffer resource of one row (raw addressing, `bytes` long): loads and stores
// then take a 32-bit per-lane byte offset plus a wave-uniform one, so a
// thread's many vectors of a row cost no per-vector 64-bit address.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The gradient of the n entries from vector offset rowv (VEC entries per
// vector): float32, or bfloat16 (GB).
template <bool GB, int VEC>
__device__ __forceinline__ Rsrc grad_rsrc(void* grad, long long rowv, int n) {
  if constexpr (GB) return row_rsrc((uint16_t*)grad + rowv * VEC, (uint32_t)n * 2u);
  else return row_rsrc((float*)grad + rowv * VEC, (uint32_t)n * 4u);
}

template <int VAR>
struct Tr;

template <>
struct Tr<kBf16x8> {  // 8 bfloat16 per 16-byte load
  static constexpr int VEC = 8, NVMAX = 8, EB = 2;
  using S = u32x4;
  __device__ static const void* row(const void* base, long long r) { return (const u32x4*)base + r; }
  __device__ static S load(const void* row, unsigned vi) { return ((const u32x4*)row)[vi]; }
  template <int AUX = 0>
  __device__ static S bload(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
  }
  // Entries 0..3 at byte voff + soff, entries 4..7 hoff bytes further (hoff
  // goes into the per-lane offset: a scalar offset the compiler cannot prove
  // uniform would make it loop over lanes).
  template <int AUX = 0>
  __device__ static S bload2(Rsrc r, uint32_t voff, uint32_t soff, uint32_t hoff) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(r, voff + hoff, soff, AUX);
    return S{a.x, a.y, b.x, b.y};
  }
  __device__ static float at(const S& s, int e) {
    const uint32_t w = s[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static float elem(const void* base, long long j) {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[j] << 16);
  }
};

template <>
struct Tr<kBf16x1> {  // one bfloat16 per access (rows not 16-byte aligned)
  static constexpr int VEC = 1, NVMAX = 16, EB = 2;
  using S = uint32_t;
  __device__ static const void* row(const void* base, long long r) { return (const uint16_t*)base + r; }
  __device__ static S load(const void* row, unsigned vi) { return ((const uint16_t*)row)[vi]; }
  template <int AUX = 0>
  __device__ static S bload(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, AUX);
  }
  __device__ static float at(const S& s, int) { return __uint_as_float(s << 16); }
  __device__ static float elem(const void* base, long long j) {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[j] << 16);
  }
};

template <>
struct Tr<kF32x4> {  // 4 float32 per 16-byte load
  static constexpr int VEC = 4, NVMAX = 8, EB = 4;
  using S = f32x4;
  __device__ static const void* row(const void* base, long long r) { return (const f32x4*)base + r; }
  __device__ static S load(const void* row, unsigned vi) { return ((const f32x4*)row)[vi]; }
  template <int AUX = 0>
  __device__ static S bload(Rsrc r, uint32_t voff, uint32_t soff) {
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    return __builtin_bit_cast(f32x4, w);
  }
  __device__ static float at(const S& s, int e) { return s[e]; }
  __device__ static float elem(const void* base, long long j) { return ((const float*)base)[j]; }
};

template <>
struct Tr<kF32x1> {
  static constexpr int VEC = 1, NVMAX = 16, EB = 4;
  using S = float;
  __device__ static const void* row(const void* base, long long r) { return (const float*)base + r; }
  __device__ static S load(const void* row, unsigned vi) { return ((const float*)row)[vi]; }
  template <int AUX = 0>
  __device__ static S bload(Rsrc r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
  }
  __device__ static float at(const S& s, int) { return s; }
  __device__ static float elem(const void* base, long long j) { return ((const float*)base)[j]; }
};

// Stores VEC gradient entries at element vi*VEC of a row (g = row start).
template <int VEC>
__device__ __forceinline__ void store_vec(float* g, unsigned vi, const float* v) {
  const unsigned off = vi * (unsigned)VEC;
  if constexpr (VEC == 8) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    const f32x4 b = {v[4], v[5], v[6], v[7]};
    store16_nt(g + off, a);
    store16_nt(g + off + 4, b);
  } else if constexpr (VEC == 4) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    store16_nt(g + off, a);
  } else {
    __builtin_nontemporal_store(v[0], g + off);
  }
}

// bfloat16 gradient output: each float32 entry rounded to nearest, ties to
// even (the hardware's packed conversion in the default rounding mode), two
// per 32-bit word, lower index in the low half.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
__device__ __forceinline__ uint32_t bf16_rne(float x) { return pack_bf16(x, 0.0f) & 0xFFFFu; }

// Stores VEC bfloat16 gradient entries at element vi*VEC of a row.
template <int VEC>
__device__ __forceinline__ void store_vec_bf16(uint16_t* g, unsigned vi, const float* v) {
  const unsigned off = vi * (unsigned)VEC;
  if constexpr (VEC == 8) {
    const u32x4 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                     pack_bf16(v[6], v[7])};
    __builtin_nontemporal_store(w, (u32x4*)(g + off));
    settle16(w);
  } else if constexpr (VEC == 4) {
    const u32x2 w = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    __builtin_nontemporal_store(w, (u32x2*)(g + off));
  } else {
    __builtin_nontemporal_store((uint16_t)bf16_rne(v[0]), g + off);
  }
}

// Same through a row's buffer resource: VEC entries at byte offset voff + soff.
// Cache policy (buffer instruction aux bits) of the logit loads.  Data read
// once (held on chip, or only scanned for the argmax) and the second read of
// the streamed part of a verified row are nontemporal; the first read of the
// streamed part is not, so that its second read can hit in cache.
#ifndef AV_AUX_RES
#define AV_AUX_RES 2
#endif
#ifndef AV_AUX_STR
#define AV_AUX_STR 0
#endif
#ifndef AV_AUX_RE
#define AV_AUX_RE 2
#endif
constexpr int kAuxOnce = AV_AUX_RES, kAuxFirst = AV_AUX_STR, kAuxAgain = AV_AUX_RE;

// Cache policy of the gradient stores (buffer instruction aux bits).
#ifndef AV_STORE_AUX
#define AV_STORE_AUX 2  // nontemporal: the gradient is not read again by this pass
#endif
constexpr int kStoreAux = AV_STORE_AUX;

template <int VEC>
__device__ __forceinline__ void bstore_vec(Rsrc g, uint32_t voff, uint32_t soff, const float* v) {
  constexpr int kNT = kStoreAux;
  if constexpr (VEC == 8) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    const f32x4 b = {v[4], v[5], v[6], v[7]};
    bstore16<kNT>(__builtin_bit_cast(u32x4, a), g, voff, soff);
    bstore16<kNT>(__builtin_bit_cast(u32x4, b), g, voff + 16u, soff);
  } else if constexpr (VEC == 4) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    bstore16<kNT>(__builtin_bit_cast(u32x4, a), g, voff, soff);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), g, voff, soff, kNT);
  }
}

// ---------------------------------------------------------------------------
// per-entry math shared by the fused and the standalone backward pass
// ---------------------------------------------------------------------------

// Tempered form (TM): the reverse-KL term compares softmax(zp / T) with
// softmax(zq / T); s = 1 / T and sL = log2(e) / T scale the logits there,
// lse_p and lse_q are the log-sum-exps of the scaled rows, and the hard
// cross-entropy keeps the plain softmax of zq (its log-sum-exp lse_q1).
struct RowK {
  float lseqL, delta, tau, s, sL;
};
template <bool TM>
__device__ __forceinline__ RowK row_consts(float lse_p, float lse_q, float tau, float s, float sL) {
  RowK k;
  k.lseqL = lse_q * kLog2e;
  k.delta = lse_q - lse_p;
  k.tau = tau;
  k.s = TM ? s : 1.0f;
  k.sL = TM ? sL : kLog2e;
  return k;
}
// q_j = exp(s zq_j - lse_q); r_j = q_j ell_j = q_j (log q_j - log p_j), with
// the log-ratio ell_j formed from the logits, s (zq_j - zp_j) - (lse_q - lse_p).
template <bool TM>
__device__ __forceinline__ void opd_entry(float zp, float zq, const RowK& k, float& q, float& ell,
                                          float& r) {
  q = __builtin_amdgcn_exp2f(__builtin_fmaf(zq, TM ? k.sL : kLog2e, -k.lseqL));
  ell = TM ? __builtin_fmaf(k.s, zq - zp, -k.delta) : (zq - zp) - k.delta;
  r = q * ell;
}

// d loss / d zq_j = gs [lam (q1_j - [j = a]) + (1 - lam) s (g_j - S q_j)]
// (q1 = softmax(zq); at T = 1, q1 = q and s = 1) with g_j = q_j (ell_j + 1)
// where |r_j| <= tau and 0 elsewhere, formed as
//   T = 1:  q_j t_j - [j = a] gs lam,
//   TM:     C1 q1_j + q_j t_j - [j = a] gs lam,
//   t_j = A + B + B ell_j where |r_j| <= tau, A elsewhere,
//   A = gs (lam - (1 - lam) S) (T = 1) or -gs (1 - lam) s S (TM), B = gs (1 - lam) s.
// With ell_j = s d_j - delta (d_j = zq_j - zp_j, delta = lse_q - lse_p), the
// inside value is taken as t_j = Bs d_j + C0 (Bs = B s at T != 1, B at T = 1;
// C0 = A + B - B delta, rounded once): one operation fewer per entry.
struct GradK {
  float a, ab, b, fix, c1, l1L, bd, c0;
};
template <bool TM>
__device__ __forceinline__ GradK grad_consts(float lam, float gs, float S, float s, float lse1, float delta) {
  GradK g;
  if constexpr (TM) {
    g.b = gs * (1.0f - lam) * s;
    g.a = -g.b * S;
    g.c1 = gs * lam;
    g.l1L = lse1 * kLog2e;
  } else {
    g.a = gs * (lam - (1.0f - lam) * S);
    g.b = gs * (1.0f - lam);
    g.c1 = 0.0f;
    g.l1L = 0.0f;
  }
  g.ab = g.a + g.b;
  g.fix = gs * lam;
  g.bd = TM ? g.b * s : g.b;
  g.c0 = __builtin_fmaf(-g.b, delta, g.ab);
  return g;
}
template <bool TM>
__device__ __forceinline__ float grad_entry(float q, float d, float r, float zq, float tau, const GradK& c) {
  const float t = (__builtin_fabsf(r) <= tau) ? __builtin_fmaf(c.bd, d, c.c0) : c.a;
  if constexpr (TM)
    return __builtin_fmaf(c.c1, __builtin_amdgcn_exp2f(__builtin_fmaf(zq, kLog2e, -c.l1L)), q * t);
  return q * t;
}
// The same for an entry known to lie inside the clip interval.
template <bool TM>
__device__ __forceinline__ float grad_entry_inside(float q, float d, float zq, const GradK& c) {
  const float t = __builtin_fmaf(c.bd, d, c.c0);
  if constexpr (TM)
    return __builtin_fmaf(c.c1, __builtin_amdgcn_exp2f(__builtin_fmaf(zq, kLog2e, -c.l1L)), q * t);
  return q * t;
}

// ---------------------------------------------------------------------------
// fused pass: one 1024-thread workgroup per row
// ---------------------------------------------------------------------------

constexpr int kRowWaves = kRowBlock / 64;
static_assert(kRowWaves == 16, "the second-level reductions take 16 wave partials in lanes 0-15");
constexpr int kLastWave = kRowWaves - 1;  // publishes rows and finishes requests
// Floor of the factor that rescales the clip-bound maxima when a thread's
// running max of zq grows: keeps them upper bounds instead of letting them
// underflow (an entry that small relative to the max has q_j |ell_j| far
// below any tau for finite logits).
constexpr float kRescaleFloor = 0x1p-100f;
// A region whose bound on q_j |ell_j| stays below this fraction of tau needs
// no entry-by-entry clip check.  The bound and the gradient pass's r_j carry
// float32 rounding of order 1e-5 relative; the 1% margin covers it many times
// over, so no entry of a certified region can reach the interval's edge.
constexpr float kClipCertify = 0.99f;
// Temperature-1 sums are rescaled only when a logit passes their reference by
// more than this (natural-log units): every term exp(z - ref) stays below
// e^11 < 2^16, so a thread's float32 sums cannot overflow, and the rounding
// of exponents up to 16 (log2 units) is under 1e-6 relative per term.
constexpr float kLazyGap = 11.0f;

template <int VAR>
struct RowCfg {  // vectors per thread kept in registers (NR) and in LDS (NL)
  static constexpr bool kWide = VAR == kBf16x8 || VAR == kF32x4;
  static constexpr int NR = kWide ? kRowRegs16 : kRowRegs1;
  static constexpr int NL = kWide ? kRowLds16 : kRowLds1;
};

// Workgroup state.  Per-wave partials and the claimed item are double-buffered
// by the parity of the row iteration.  Every row passes at least one barrier,
// so a buffer is rewritten two rows later only after every wave has read it,
// and the waves need not meet at the start of a row: a wave that is done with
// one row's gradient starts loading the next row.
struct RowSmem {
  float f[2][kRowWaves][6];   // mp, sp, mq, sq, kq, zq at the argmax
  int i[2][kRowWaves];        // first index of mp
  double d[2][kRowWaves][2];  // clip corrections of S and of the KL sum
  uint64_t item[2];           // claimed dispenser word (status bits << 32 | item)
  int hist[AV_MAX_K + 1];     // longest-first schedule of the dense layout:
  int cnt[AV_MAX_K + 1];      //   requests with b_k > p
  int cum[AV_MAX_K + 1];      //   verified rows at positions < p
  int cumu[AV_MAX_K + 1];     //   unverified rows at positions < p
  uint64_t exitw;
  uint32_t tag;
  float f1[2][kRowWaves];     // tempered form: sq1
};

// Running statistics of one thread's part of a row.
struct RowAcc {
  float mp, sp;  // max of zp, sum exp(zp - mp)
  int bi;        // first index of mp
  float za;      // zq at that index
  float mq, sq;  // max of zq, sum exp(zq - mq)
  float kq;      // sum exp(zq - mq) (zq - zp): the reverse KL, once normalised
  float sq1;     // tempered form: sum exp(zq - mq) at temperature 1 (the sums
                 // above then scale exponents by 1 / T; kq's difference does not)
  float rp;      // reference of sp (sp = sum exp((zp - rp) / T)), see kLazyGap
  float mq_on, mq_st;  // per region (on chip / streamed): max zq
  float pm_on, pm_st;  // per region: max exp(zq - mq) |zq - zp| (mq: running max)
};

__device__ __forceinline__ void acc_init(RowAcc& A) {
  A.mp = -INFINITY;
  A.sp = 0.0f;
  A.rp = -INFINITY;
  A.bi = INT_MAX;
  A.za = 0.0f;
  A.mq = -INFINITY;
  A.sq = 0.0f;
  A.kq = 0.0f;
  A.sq1 = 0.0f;
  A.mq_on = -INFINITY;
  A.mq_st = -INFINITY;
  A.pm_on = 0.0f;
  A.pm_st = 0.0f;
}

// Index of entry e of a vector whose entries 0..3 are consecutive from lo
// and entries 4..7 consecutive from lo + H (H = 4: one consecutive run).
__device__ __forceinline__ int entry_index(int lo, int H, int e) {
  return e < 4 ? lo + e : lo + H + (e - 4);
}

// Folds one vector (entries at lo.., lo+H..) into the running statistics
// (online normaliser: sums are rescaled when a larger maximum appears).
// `onchip` selects the clip-bound region of the vector.  TM: exponents are
// scaled by sL = log2(e) / T, and sq1 sums the unscaled ones; they are formed
// as (z - max) sL, whose only rounding is that of a product that vanishes at
// the maximum (z sL - max sL would round max sL, which grows like 1 / T, and
// scale every term of the thread by that error).
template <int VAR, bool TM>
__device__ __forceinline__ void acc_vec(const typename Tr<VAR>::S& xp, const typename Tr<VAR>::S& xq,
                                        int lo, int H, RowAcc& A, bool onchip, float sL,
                                        float gp = kLazyGap, float gq = kLazyGap) {
  using T = Tr<VAR>;
  constexpr int VEC = T::VEC;
  const float L = TM ? sL : kLog2e;
  float vp = T::at(xp, 0), vq = T::at(xq, 0);
#pragma unroll
  for (int e = 1; e < VEC; ++e) {
    vp = fmaxf(vp, T::at(xp, e));
    vq = fmaxf(vq, T::at(xq, e));
  }
  if (__builtin_expect(vp >= A.mp, 0)) {  // may hold a new first maximum
    int e0 = VEC - 1;
    float z0 = T::at(xq, VEC - 1);
#pragma unroll
    for (int e = VEC - 2; e >= 0; --e)  // entry order is index order
      if (T::at(xp, e) == vp) {
        e0 = e;
        z0 = T::at(xq, e);
      }
    const int idx = entry_index(lo, H, e0);
    if (vp > A.mp || idx < A.bi) {
      A.bi = idx;
      A.za = z0;
    }
  }
  const float np = fmaxf(A.mp, vp);
  if constexpr (!TM) {
    // Temperature 1: the sums keep their references (rp for zp, mq for zq)
    // until a value passes one by more than kLazyGap; only then (rarely, for
    // the whole wave at once) are they rescaled, to the running maxima.
    A.mp = np;
    if (__builtin_expect(__any(vp > A.rp + kLazyGap || vq > A.mq + kLazyGap), 0)) {
      A.sp *= __builtin_amdgcn_exp2f((A.rp - np) * kLog2e);
      A.rp = np;
      const float nq = fmaxf(A.mq, vq);
      const float sc = __builtin_amdgcn_exp2f((A.mq - nq) * kLog2e);
      A.sq *= sc;
      A.kq *= sc;
      const float scb = fmaxf(sc, kRescaleFloor);
      A.pm_on *= scb;
      A.pm_st *= scb;
      A.mq = nq;
    }
    const float rpL = A.rp * kLog2e, rqL = A.mq * kLog2e;
    float pm = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float q = T::at(xq, e), p = T::at(xp, e);
      A.sp += __builtin_amdgcn_exp2f(__builtin_fmaf(p, kLog2e, -rpL));
      const float eq = __builtin_amdgcn_exp2f(__builtin_fmaf(q, kLog2e, -rqL));
      const float d = q - p;
      A.sq += eq;
      A.kq = __builtin_fmaf(eq, d, A.kq);
      pm = fmaxf(pm, eq * __builtin_fabsf(d));
    }
    if (onchip) {
      A.mq_on = fmaxf(A.mq_on, vq);
      A.pm_on = fmaxf(A.pm_on, pm);
    } else {
      A.mq_st = fmaxf(A.mq_st, vq);
      A.pm_st = fmaxf(A.pm_st, pm);
    }
    return;
  }
  // Tempered: the same lazy references, with gaps in logit units: gp keeps
  // every term of sp and sq below exp(kLazyGap) (gp = kLazyGap T), gq also
  // those of sq1, whose exponents are not scaled (gq = min(gp, kLazyGap)).
  A.mp = np;
  if (__builtin_expect(__any(vp > A.rp + gp || vq > A.mq + gq), 0)) {
    A.sp *= __builtin_amdgcn_exp2f((A.rp - np) * L);
    A.rp = np;
    const float nq = fmaxf(A.mq, vq);
    const float sc = __builtin_amdgcn_exp2f((A.mq - nq) * L);
    A.sq *= sc;
    A.kq *= sc;
    A.sq1 *= __builtin_amdgcn_exp2f((A.mq - nq) * kLog2e);
    const float scb = fmaxf(sc, kRescaleFloor);
    A.pm_on *= scb;
    A.pm_st *= scb;
    A.mq = nq;
  }
  const float rp = A.rp, rq = A.mq;
  float pm = 0.0f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float q = T::at(xq, e), p = T::at(xp, e);
    A.sp += __builtin_amdgcn_exp2f((p - rp) * L);
    const float dq = q - rq;
    const float eq = __builtin_amdgcn_exp2f(dq * L);
    A.sq1 += __builtin_amdgcn_exp2f(dq * kLog2e);
    const float d = q - p;
    A.sq += eq;
    A.kq = __builtin_fmaf(eq, d, A.kq);
    pm = fmaxf(pm, eq * __builtin_fabsf(d));
  }
  if (onchip) {
    A.mq_on = fmaxf(A.mq_on, vq);
    A.pm_on = fmaxf(A.pm_on, pm);
  } else {
    A.mq_st = fmaxf(A.mq_st, vq);
    A.pm_st = fmaxf(A.pm_st, pm);
  }
}

// (m, s) <- log-sum-exp merge; commutative, so xor butterflies leave the same
// bits in every lane.  Empty parts (s == 0) contribute nothing.
// L scales the exponents (log2(e), or log2(e) / T for tempered sums).
__device__ __forceinline__ void lse_merge(float& m, float& s, float& k, float om, float os,
                                          float ok, float L = kLog2e) {
  const float M = fmaxf(m, om);
  const float fa = (s == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((m - M) * L);
  const float fb = (os == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((om - M) * L);
  m = M;
  s = s * fa + os * fb;
  k = k * fa + ok * fb;
}

// Lane 0's value in every lane, through a scalar register (every lane of
// the wave must be active, so that lane 0 is the first active one).
__device__ __forceinline__ uint32_t bcast0(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ int bcast0(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float bcast0(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ double bcast0(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = bcast0((uint32_t)b), hi = bcast0((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Lane l's value, through a scalar register.
__device__ __forceinline__ int lane_of(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_of(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_of(double v, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Reductions of the fused row kernel, in two stages.  Inside each row of 16
// lanes, four DPP moves pair every lane with another (neighbours, pairs of a
// quad, mirror images in 8 lanes, mirror images in 16) and each step combines
// the two values with a commutative operation, so after the four steps every
// lane of a row holds the row's result with the same bits.  The four rows'
// results are then read into scalar registers and combined in row order.
// NL = 16: only lanes 0-15 hold values, and the result is row 0's.  Every
// lane of the wave must be active.
constexpr int kDppSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppMirror8 = 0x141;  // row_half_mirror
constexpr int kDppMirror16 = 0x140; // row_mirror
template <int C>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, C, 0xF, 0xF, false);
}
template <int C>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(dpp<C>(__float_as_int(v)));
}
template <int C>
__device__ __forceinline__ double dpp(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp<C>((int)(uint32_t)b), hi = (uint32_t)dpp<C>((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <class T>
__device__ __forceinline__ T row_sum(T v) {
  v += dpp<kDppSwap1>(v);
  v += dpp<kDppSwap2>(v);
  v += dpp<kDppMirror8>(v);
  v += dpp<kDppMirror16>(v);
  return v;
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<kDppSwap1>(v));
  v = fmaxf(v, dpp<kDppSwap2>(v));
  v = fmaxf(v, dpp<kDppMirror8>(v));
  v = fmaxf(v, dpp<kDppMirror16>(v));
  return v;
}
template <int NL, class T>
__device__ __forceinline__ T xsum(T v) {
  v = row_sum(v);
  if constexpr (NL == 16) return bcast0(v);
  else return (lane_of(v, 0) + lane_of(v, 16)) + (lane_of(v, 32) + lane_of(v, 48));
}
template <int NL>
__device__ __forceinline__ float xmax(float v) {
  v = row_max(v);
  if constexpr (NL == 16) return bcast0(v);
  else return fmaxf(fmaxf(lane_of(v, 0), lane_of(v, 16)), fmaxf(lane_of(v, 32), lane_of(v, 48)));
}
// Smallest index, with the value that goes with it.
template <int C>
__device__ __forceinline__ void min_step(int& i, float& z) {
  const int oi = dpp<C>(i);
  const float oz = dpp<C>(z);
  if (oi < i) {
    i = oi;
    z = oz;
  }
}
template <int NL>
__device__ __forceinline__ void xminidx(int& i, float& z) {
  min_step<kDppSwap1>(i, z);
  min_step<kDppSwap2>(i, z);
  min_step<kDppMirror8>(i, z);
  min_step<kDppMirror16>(i, z);
  if constexpr (NL == 16) {
    i = bcast0(i);
    z = bcast0(z);
  } else {
    int bi = lane_of(i, 0);
    float bz = lane_of(z, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const int oi = lane_of(i, 16 * r);
      const float oz = lane_of(z, 16 * r);
      if (oi < bi) {
        bi = oi;
        bz = oz;
      }
    }
    i = bi;
    z = bz;
  }
}
// (value desc, index asc): the first index of the largest value.
template <int C>
__device__ __forceinline__ void amax_step(float& v, int& i) {
  amax_merge(v, i, dpp<C>(v), dpp<C>(i));
}
template <int NL>
__device__ __forceinline__ void xargmax(float& v, int& i) {
  amax_step<kDppSwap1>(v, i);
  amax_step<kDppSwap2>(v, i);
  amax_step<kDppMirror8>(v, i);
  amax_step<kDppMirror16>(v, i);
  if constexpr (NL == 16) {
    v = bcast0(v);
    i = bcast0(i);
  } else {
    float bv = lane_of(v, 0);
    int bi = lane_of(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) amax_merge(bv, bi, lane_of(v, 16 * r), lane_of(i, 16 * r));
    v = bv;
    i = bi;
  }
}

// A wave's row statistics combined by one pass of maxima, one rescale of each
// lane's sums and one pass of sums (instead of a log-sum-exp merge at each
// reduction step).  On entry sp is relative to mp; on exit every lane holds
// the same bits: the wave's max of zp, its first index and the zq there, the
// sums relative to the wave's maxima, and kq.  Lanes with empty sums
// contribute nothing.  TM: sp, sq and kq scale exponents by L = log2(e) / T,
// sq1 (temperature 1) does not.  NL = 16: only lanes 0-15 hold partials.
template <bool TM, int NL = 64>
__device__ __forceinline__ void wave_combine(RowAcc& W, float L = kLog2e) {
  const float M = xmax<NL>(W.mp);
  int bi = (W.mp == M) ? W.bi : INT_MAX;
  float za = W.za;
  xminidx<NL>(bi, za);
  const float sp = (W.sp == 0.0f) ? 0.0f : W.sp * __builtin_amdgcn_exp2f((W.mp - M) * L);
  const float Mq = xmax<NL>(W.mq);
  const float f = (W.sq == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((W.mq - Mq) * L);
  if constexpr (TM) {
    const float f1 = (W.sq1 == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((W.mq - Mq) * kLog2e);
    W.sq1 = xsum<NL>(W.sq1 * f1);
  }
  W.sp = xsum<NL>(sp);
  W.sq = xsum<NL>(W.sq * f);
  W.kq = xsum<NL>(W.kq * f);
  W.mp = M;
  W.rp = M;
  W.bi = bi;
  W.za = za;
  W.mq = Mq;
}

// Sum of the first 16 lanes, the same bits in every lane (all lanes active).
__device__ __forceinline__ double wsumd16(double v) { return xsum<16>(v); }

// Claims the next dispense index; the high half carries the launch's status.
// Number of zero bytes of x (exact: no carry crosses a byte).
__device__ __forceinline__ int zero_bytes(uint64_t x) {
  const uint64_t t = ((x & 0x7f7f7f7f7f7f7f7full) + 0x7f7f7f7f7f7f7f7full) | x;
  return __popcll(~t & 0x8080808080808080ull);
}

__device__ __forceinline__ uint64_t claim(const FwdArgs& a) {
  return __hip_atomic_fetch_add(a.ctl, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts one more completed row of a request; returns the new count.  The
// counter word is {tag, count}: a word from an earlier launch counts as 0.
// One fetch-and-add when the word already carries this launch's tag (every
// arrival but a request's first); otherwise the add only touched a stale
// word, which counts as 0 whatever it holds (a carry into its tag included),
// and a compare-and-swap loop takes the word over.
__device__ __forceinline__ uint32_t arrive(uint64_t* p, uint32_t tag) {
  uint64_t old = __hip_atomic_fetch_add(p, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tag_ok(old, tag)) return (uint32_t)old + 1u;
  old = tget(p);
  for (;;) {
    const uint32_t n = tag_ok(old, tag) ? (uint32_t)old + 1u : 1u;
    const uint64_t nw = ((uint64_t)tag << 32) | (uint64_t)n;
    if (__hip_atomic_compare_exchange_strong(p, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return n;
  }
}

// Work item: a row, its request, and whether it is verified.
struct Item {
  int row, req, r0, bkb;  // r0: first row of the request; bkb: its verified rows
  int half;               // unverified rows in parts: the part (0 .. nparts-1); else -1
  int nparts;             // 2 (halves) or 4 (quarters)
  bool verified;
};

// Dense layout, longest first: verified rows position-major (position p holds
// the cnt[p] requests with b_k > p, which lead `order`, sorted by b_k
// descending), then unverified rows position-major (the requests with
// b_k <= p, which trail `order`), each as two halves and the last nq of them
// as four quarters, so that the last work items of a launch are short.
// whole: unverified rows are one item each (split rows: the pair's two
// workgroups take their halves).
__device__ __forceinline__ Item map_item(const FwdArgs& a, const RowSmem& sm, const int* s_off,
                                         const uint16_t* order, const uint8_t* key, int idx,
                                         bool whole, int nq = 0) {
  Item m;
  m.nparts = 2;
  if (a.ragged) {
    int lo = 0, hi = opaque_s(a.B) - 1;  // last request whose first row is <= idx
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= idx) lo = mid;
      else hi = mid - 1;
    }
    m.row = idx;
    m.req = lo;
    m.r0 = s_off[lo];
    m.bkb = s_off[lo + 1] - m.r0;
    m.half = -1;
    m.verified = true;
  } else if (a.lpt) {
    const int k = opaque_s(a.k), rv = sm.cum[k];
    int p, j, lo = 0, hi = k - 1;
    if (idx < rv) {
      while (lo < hi) {  // last position whose first verified row is <= idx
        const int mid = (lo + hi + 1) >> 1;
        if (sm.cum[mid] <= idx) lo = mid;
        else hi = mid - 1;
      }
      p = lo;
      j = idx - sm.cum[p];
      m.half = -1;
      m.verified = true;
    } else {
      int u;
      const int nh = 2 * (opaque_s(a.R) - rv - nq);  // items of the halved unverified rows
      if (whole) {
        u = idx - rv;
        m.half = 0;
      } else if (idx - rv < nh) {
        u = (idx - rv) >> 1;
        m.half = (idx - rv) & 1;
      } else {
        u = (nh >> 1) + ((idx - rv - nh) >> 2);
        m.half = (idx - rv - nh) & 3;
        m.nparts = 4;
      }
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sm.cumu[mid] <= u) lo = mid;
        else hi = mid - 1;
      }
      p = lo;
      j = sm.cnt[p] + (u - sm.cumu[p]);
      m.verified = false;
    }
    m.req = order[j];
    m.r0 = m.req * k;
    m.row = m.r0 + p;
    m.bkb = key[m.req];
  } else {
    m.row = idx;
    const int k = opaque_s(a.k);
    m.req = idx / k;
    m.r0 = m.req * k;
    m.bkb = min(max(a.bk[m.req], 1), k);
    m.half = whole ? 0 : -1;
    m.verified = idx - m.r0 < m.bkb;
  }
  return m;
}

// The launch's arguments, read from the kernel-argument segment at the point
// of use.  The fused kernel's rarely used fields (output and workspace
// pointers of the per-row and per-request results) go through this, so they
// do not occupy scalar registers across the row loop.
typedef const __attribute__((address_space(4))) FwdArgs* KArgs;
__device__ __forceinline__ KArgs cold_args() {
  KArgs p = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// Request `req` (rows r0 .. r0+bkb-1 verified) is complete: accepted length
// and request loss.  Run by one wave of the workgroup that counted the
// request's last row; the other rows' words carry the tag once visible.
__device__ __forceinline__ void finish_request(const FwdArgs& a, int req, int r0, int bkb,
                                               uint32_t tag) {
  const int lane = threadIdx.x & 63;
  const KArgs K = cold_args();
  uint64_t w0 = 0, w1 = 0;
  Waiter wt(a.ctl, K->timeout_ticks);
  for (;;) {
    bool ok = true;
    if (lane < bkb) {
      w0 = tget(K->rowres + 2 * (long long)(r0 + lane));
      w1 = tget(K->rowres + 2 * (long long)(r0 + lane) + 1);
      ok = tag_ok(w0, tag) && tag_ok(w1, tag);
    }
    if (__all(ok)) break;
    if (!__all(wt.keep_going())) break;
  }
  const bool inb = lane < bkb;
  bool match = false;
  if (inb) match = K->draft[r0 + lane] == (int32_t)(uint32_t)w0;
  const uint64_t mism = __ballot(inb && !match);
  const int acc = mism ? (__ffsll((unsigned long long)mism) - 1) : bkb;
  double v = inb ? (double)lo_f(w1) : 0.0;
  v = xsum<64>(v);
  if (lane == 0) {
    K->acc[req] = acc;
    if (K->req_loss) K->req_loss[req] = (float)v;
    const uint64_t bits = (uint64_t)__double_as_longlong(v);
    tput(K->reqres + 2 * (long long)req, tag, (uint32_t)(bits >> 32));
    tput(K->reqres + 2 * (long long)req + 1, tag, (uint32_t)bits);
  }
}

// Sum of the request losses in a fixed order; run by the workgroup that
// leaves last, when every request has been finished.  False on a timeout.
__device__ __forceinline__ bool finish_total(const FwdArgs& a, RowSmem& sm, uint32_t tag) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const KArgs K = cold_args();
  double part = 0.0;
  bool ok = true;
  for (int b = tid; b < a.B; b += kRowBlock) {
    uint64_t h = 0, l = 0;
    Waiter wt(a.ctl, K->timeout_ticks);
    for (;;) {
      h = tget(K->reqres + 2 * (long long)b);
      l = tget(K->reqres + 2 * (long long)b + 1);
      if (tag_ok(h, tag) && tag_ok(l, tag)) break;
      if (!wt.keep_going()) {
        ok = false;
        break;
      }
    }
    part += __longlong_as_double((long long)(((uint64_t)(uint32_t)h << 32) | (uint32_t)l));
  }
  part = xsum<64>(part);
  if (lane == 0) sm.d[0][wid][0] = part;
  ok = __syncthreads_and(ok);
  if (wid == 0) {
    double t = (lane < kRowWaves) ? sm.d[0][lane][0] : 0.0;
    t = wsumd16(t);
    if (lane == 0 && K->total) K->total[0] = (float)t;
  }
  return ok;
}

// Per-thread access pattern of a row in the fused pass.
//
// A row is split into slots of kRowBlock vectors; wave w of the workgroup
// owns vectors w*64 .. w*64+63 of every slot (a "wave block").  For 16-byte
// float32 vectors and for scalars, lane l owns vector w*64 + l: consecutive
// entries.  For bfloat16 rows (8 entries per vector) lane l owns entries
// 4l..4l+3 of the first half of its wave block and the same four of the
// second half (a block of n vectors has halves of 4n entries), so each
// 16-byte gradient store of a wave covers one contiguous stretch of memory
// (stores that each fill only half of every 32 bytes double the HBM write
// traffic).
template <int VAR>
struct RowIO {
  using T = Tr<VAR>;
  using S = typename T::S;
  static constexpr bool kHalves = VAR == kBf16x8;
  static constexpr int VEC = T::VEC;
  static constexpr uint32_t SIN = kRowBlock * VEC * T::EB;  // bytes of logits per slot
  static constexpr uint32_t SOUT = kRowBlock * VEC * 4u;    // bytes of gradient per slot
  static constexpr int SE = kRowBlock * VEC;                // entries per slot
  int wid, lane;
  uint32_t voff, goff;  // byte offsets of the thread's first load / store in slot 0
  int lo0;              // row index of the thread's entry 0 in slot 0

  // ebase: row index of the first entry (a split row's second half starts
  // inside the row).
  __device__ __forceinline__ explicit RowIO(int tid, int ebase = 0) {
    wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    if constexpr (kHalves) {
      voff = (uint32_t)(wid * 64 * VEC * T::EB + lane * 4 * T::EB);
      goff = (uint32_t)(wid * 64 * VEC * 4 + lane * 16);
      lo0 = ebase + wid * 64 * VEC + lane * 4;
    } else {
      voff = (uint32_t)(tid * VEC * T::EB);
      goff = (uint32_t)(tid * VEC * 4);
      lo0 = ebase + tid * VEC;
    }
  }
  // Vectors of the wave's block in slot s (wave-uniform; 64 unless the block
  // crosses the end of the row).
  __device__ __forceinline__ int nb(int s, int nvec) const {
    const int n = nvec - s * kRowBlock - wid * 64;
    return n < 0 ? 0 : (n > 64 ? 64 : n);
  }
  __device__ __forceinline__ bool has(int nbv) const { return lane < nbv; }
  __device__ __forceinline__ int lo(int s) const { return lo0 + s * SE; }
  __device__ __forceinline__ int H(int nbv) const { return kHalves ? 4 * nbv : 4; }
  template <int AUX = 0>
  __device__ __forceinline__ S load(Rsrc r, int s, int nbv) const {
    if constexpr (kHalves)
      return T::template bload2<AUX>(r, voff, (uint32_t)s * SIN, (uint32_t)(nbv * 4 * T::EB));
    else return T::template bload<AUX>(r, voff, (uint32_t)s * SIN);
  }
  // The thread's vector from an LDS slot filled by direct loads (lane l's
  // 16 bytes at 16 l of the wave's part: the block's entries in order).
  __device__ __forceinline__ S lds(const S* slot, int nbv) const {
    if constexpr (kHalves) {
      const uint64_t* w = (const uint64_t*)(slot + wid * 64);
      const uint64_t x = w[lane], y = w[lane + nbv];
      return S{(uint32_t)x, (uint32_t)(x >> 32), (uint32_t)y, (uint32_t)(y >> 32)};
    } else {
      return slot[wid * 64 + lane];
    }
  }
  // GB: bfloat16 gradient, at half the float32 byte offsets.
  template <bool GB = false>
  __device__ __forceinline__ void store(Rsrc g, int s, int nbv, const float* v) const {
    if constexpr (GB) {
      const uint32_t so = (uint32_t)s * (SOUT / 2), go = goff >> 1;
      if constexpr (VEC == 8) {  // four entries from each half of the block: 8 bytes each
        const u32x2 x = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        const u32x2 y = {pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7])};
        __builtin_amdgcn_raw_buffer_store_b64(x, g, go, so, kStoreAux);
        __builtin_amdgcn_raw_buffer_store_b64(y, g, go + (uint32_t)nbv * 8u, so, kStoreAux);
      } else if constexpr (VEC == 4) {
        const u32x2 x = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(x, g, go, so, kStoreAux);
      } else {
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)bf16_rne(v[0]), g, go, so, kStoreAux);
      }
    } else if constexpr (kHalves) {
      const f32x4 x = {v[0], v[1], v[2], v[3]};
      const f32x4 y = {v[4], v[5], v[6], v[7]};
      const uint32_t so = (uint32_t)s * SOUT;
      bstore16<kStoreAux>(__builtin_bit_cast(u32x4, x), g, goff, so);
      bstore16<kStoreAux>(__builtin_bit_cast(u32x4, y), g, goff + (uint32_t)nbv * 16u, so);
    } else {
      bstore_vec<VEC>(g, goff, (uint32_t)s * SOUT, v);
    }
  }
};

// Folds one zp vector of consecutive entries into a running (max, first
// index) pair; vectors come in increasing order, so a strict > keeps the first.
template <int VAR>
__device__ __forceinline__ void argmax_vec(const typename Tr<VAR>::S& x, int vi, float& m, int& bi) {
  using T = Tr<VAR>;
  constexpr int VEC = T::VEC;
  float vm = T::at(x, 0);
#pragma unroll
  for (int e = 1; e < VEC; ++e) vm = fmaxf(vm, T::at(x, e));
  if (vm > m) {
    int e0 = VEC - 1;
#pragma unroll
    for (int e = VEC - 2; e >= 0; --e)
      if (T::at(x, e) == vm) e0 = e;
    m = vm;
    bi = vi * VEC + e0;
  }
}

// Zero gradient of slots [s0, s1) of a row (16-byte pieces where the row
// allows them; a slot is kRowBlock pieces).
template <int VAR, bool GB>
__device__ __forceinline__ void zero_slots(const FwdArgs& a, long long rowv, int tid, int s0, int s1) {
  constexpr int VEC = Tr<VAR>::VEC;
  const int V = opaque_s(a.V);
  const Rsrc g = grad_rsrc<GB, VEC>(a.grad, rowv, V);
  const u32x4 z = {0u, 0u, 0u, 0u};
  if constexpr (GB) {  // bfloat16 zeros: the same slots, in 8-byte pieces (4 entries)
    const u32x2 z2 = {0u, 0u};
    const int n4 = V / 4;
    const uint32_t off = (uint32_t)tid * 8u;
    if constexpr (VEC >= 4) {
#pragma unroll 4
      for (int s = s0; s < s1; ++s)
        if (s * kRowBlock + tid < n4)
          __builtin_amdgcn_raw_buffer_store_b64(z2, g, off, (uint32_t)s * (kRowBlock * 8u), kStoreAux);
    } else {
      const uint32_t off1 = (uint32_t)tid * 2u;
#pragma unroll 4
      for (int s = s0; s < s1; ++s)
        if (s * kRowBlock + tid < V)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, g, off1, (uint32_t)s * (kRowBlock * 2u), kStoreAux);
    }
  } else if constexpr (VEC >= 4) {
    const int n4 = V / 4;  // 16-byte pieces per row
    const uint32_t off = (uint32_t)tid * 16u;
#pragma unroll 4
    for (int s = s0; s < s1; ++s)
      if (s * kRowBlock + tid < n4) bstore16<kStoreAux>(z, g, off, (uint32_t)s * (kRowBlock * 16u));
  } else {
    const uint32_t off = (uint32_t)tid * 4u;
#pragma unroll 4
    for (int s = s0; s < s1; ++s)
      if (s * kRowBlock + tid < V)
        __builtin_amdgcn_raw_buffer_store_b32(0u, g, off, (uint32_t)s * (kRowBlock * 4u), kStoreAux);
  }
}

// Unverified row (half < 0) or part `half` of np parts of one: target argmax
// only, zero gradient.  Part h covers the h-th of np runs of the row's vector
// slots and of its gradient's 16-byte slots; the part that completes the row
// last merges the np maxima (the lower index wins ties) and writes the
// results.
template <int VAR, bool GB>
__device__ __forceinline__ void unverified_row(const FwdArgs& a, RowSmem& sm, int row, int par, int half,
                                               int np, uint32_t tag) {
  using T = Tr<VAR>;
  constexpr int VEC = T::VEC;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wid = tid >> 6;
  uint64_t nxt = 0;
  if (tid == 0) nxt = claim(a);  // answered with this row's first loads
  const long long rowv = (long long)row * a.nvec;
  const Rsrc rzp = row_rsrc(T::row(a.zp, rowv), (uint32_t)opaque_s(a.V) * (uint32_t)T::EB);
  constexpr uint32_t VB = T::VEC * T::EB, SIN = kRowBlock * VB;
  const uint32_t voff = (uint32_t)tid * VB;
  const int nvec = opaque_s(a.nvec);
  const int ns = (nvec + kRowBlock - 1) / kRowBlock;       // vector slots
  const int gpieces = VEC >= 4 ? opaque_s(a.V) / 4 : opaque_s(a.V);
  const int gs = (gpieces + kRowBlock - 1) / kRowBlock;    // gradient slots
  int s0 = 0, s1 = ns, g0 = 0, g1 = gs;
  if (half >= 0) {
    s0 = ns * half / np;
    s1 = ns * (half + 1) / np;
    g0 = gs * half / np;
    g1 = gs * (half + 1) / np;
  }
  const int full_end = min(s1, nvec / kRowBlock);  // slots in which every thread has a vector
  float m = -INFINITY;
  int bi = INT_MAX;
#ifndef AV_UU
#define AV_UU 4
#endif
#pragma unroll AV_UU
  for (int s = s0; s < full_end; ++s)
    argmax_vec<VAR>(T::template bload<kAuxOnce>(rzp, voff, (uint32_t)s * SIN), s * kRowBlock + tid, m, bi);
  for (int s = max(full_end, s0); s < s1; ++s)
    if (s * kRowBlock + tid < nvec)
      argmax_vec<VAR>(T::template bload<kAuxOnce>(rzp, voff, (uint32_t)s * SIN), s * kRowBlock + tid, m, bi);
  xargmax<64>(m, bi);
  if (lane == 0) {
    sm.f[par][wid][0] = m;
    sm.i[par][wid] = bi;
  }
  if (tid == 0) sm.item[par ^ 1] = nxt;
  __syncthreads();
  if (wid == kLastWave) {
    float M = -INFINITY;
    int I = INT_MAX;
    if (lane < kRowWaves) {
      M = sm.f[par][lane][0];
      I = sm.i[par][lane];
    }
    xargmax<16>(M, I);  // the 16 wave partials sit in lanes 0-15
    bool write = half < 0;
    if (half >= 0) {  // publish this part; the last part to finish merges
      const KArgs K = cold_args();
      uint32_t n = 0;
      if (lane == 0) {
        uint64_t* hr = K->halfres + 8 * (long long)row + 2 * half;
        tput(hr, tag, __float_as_uint(M));
        tput(hr + 1, tag, (uint32_t)I);
        n = arrive(K->harrive + row, tag);
      }
      n = bcast0(n);
      if (n == (uint32_t)np) {  // lane o < np reads part o's words
        uint64_t w0 = 0, w1 = 0;
        if (lane < np && lane != half) {
          uint64_t* ho = K->halfres + 8 * (long long)row + 2 * lane;
          Waiter wt(a.ctl, K->timeout_ticks);
          for (;;) {
            w0 = tget(ho);
            w1 = tget(ho + 1);
            if (tag_ok(w0, tag) && tag_ok(w1, tag)) break;
            if (!wt.keep_going()) break;
          }
        }
        float Mo = -INFINITY;
        int Io = INT_MAX;
        if (lane < np && lane != half) {
          Mo = lo_f(w0);
          Io = (int)(uint32_t)w1;
        }
#pragma unroll
        for (int o = 0; o < 4; ++o) amax_merge(M, I, __shfl(Mo, o), __shfl(Io, o));
        write = true;
      }
    }
    if (write && lane == 0) {
      const KArgs K = cold_args();
      K->row_loss[row] = 0.0f;
      K->tgt[row] = I;
      if (K->stats) store16(K->stats + 4 * (long long)row, (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
      if (K->lse1) K->lse1[row] = 0.0f;
    }
  }
  if (a.grad) zero_slots<VAR, GB>(a, rowv, tid, g0, g1);
}

// Gradient of one vector (entries at lo.., lo+H..; the label entry Arg gets
// -gs*lam) -> store through io.  chk: the vector's region was not certified
// clip-free, so each entry's |r_j| is compared with tau; in a certified
// region every entry is inside the interval and takes the inside branch
// directly (the same float32 steps, so the same bits).  The tempered form
// always compares (measured on the concurrent workload: the shortcut made
// T = 1 0.9% and the bfloat16 gradient 2.8% faster, T = 0.5 and 2 slower).
template <int VAR, bool GB, bool TM>
__device__ __forceinline__ void grad_vec(const typename Tr<VAR>::S& xp, const typename Tr<VAR>::S& xq,
                                         const RowIO<VAR>& io, int s, int nbv, const RowK& rk,
                                         const GradK& gk, int Arg, Rsrc g, bool chk) {
  using T = Tr<VAR>;
  constexpr int VEC = T::VEC, RUN = VEC < 4 ? VEC : 4;
  float out[VEC];
  if (TM || chk) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float q, ell, r;
      opd_entry<TM>(T::at(xp, e), T::at(xq, e), rk, q, ell, r);
      out[e] = grad_entry<TM>(q, T::at(xq, e) - T::at(xp, e), r, T::at(xq, e), rk.tau, gk);
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float q, ell, r;
      opd_entry<TM>(T::at(xp, e), T::at(xq, e), rk, q, ell, r);
      out[e] = grad_entry_inside<TM>(q, T::at(xq, e) - T::at(xp, e), T::at(xq, e), gk);
    }
  }
  const int lo = io.lo(s);
  int el = -1;  // entry that holds the label, if any
  if ((unsigned)(Arg - lo) < (unsigned)RUN) el = Arg - lo;
  if constexpr (VEC == 8) {
    const int r2 = Arg - (lo + io.H(nbv));
    if ((unsigned)r2 < 4u) el = 4 + r2;
  }
  if (el >= 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      if (e == el) out[e] = out[e] - gk.fix;
  }
  io.template store<GB>(g, s, nbv, out);
}

// Row maximum of zq and log2 of its normaliser sum exp(s (zq - m)): the
// correction pass forms q_j from them.
struct FineK {
  float mq, l2s;
};

// Clip corrections of one vector: cs += (r + q) - g, ck += r - clip(r).  The
// indicator c_j is the gradient pass's (same float32 steps); the values use
// q_j = exp2((zq_j - m) sL - log2 sum), exact to a few ulp also for a dominant
// entry of a row with large logits, where the corrections nearly cancel the
// row's unclipped sums (the gradient pass's form rounds lse to float32 first).
// PRE: first the vector's own bound, exp(s max zq - lse_q) (s max |zq - zp| +
// |delta|) on q_j |ell_j| (the region bound's argument, on one vector); a
// vector below kClipCertify * tau adds nothing and is skipped.  Used for the
// on-chip vectors of the tempered form (measured at T = 0.5 on the concurrent
// workload: 457 against 473 us; at T = 1 the check made the pass slower).
template <int VAR, bool TM, bool PRE = false>
__device__ __forceinline__ void clip_vec(const typename Tr<VAR>::S& xp, const typename Tr<VAR>::S& xq,
                                         const RowK& rk, const FineK& fk, float& cs, float& ck) {
  using T = Tr<VAR>;
  if constexpr (PRE) {
    float vq = T::at(xq, 0), dm = __builtin_fabsf(T::at(xq, 0) - T::at(xp, 0));
#pragma unroll
    for (int e = 1; e < T::VEC; ++e) {
      vq = fmaxf(vq, T::at(xq, e));
      dm = fmaxf(dm, __builtin_fabsf(T::at(xq, e) - T::at(xp, e)));
    }
    const float qb = __builtin_amdgcn_exp2f(__builtin_fmaf(vq, rk.sL, -rk.lseqL));
    if (qb * __builtin_fmaf(rk.s, dm, __builtin_fabsf(rk.delta)) <= kClipCertify * rk.tau) return;
  }
#pragma unroll
  for (int e = 0; e < T::VEC; ++e) {
    const float zp = T::at(xp, e), zq = T::at(xq, e);
    float q, ell, r;
    opd_entry<TM>(zp, zq, rk, q, ell, r);
    const float qf = __builtin_amdgcn_exp2f(__builtin_fmaf(zq - fk.mq, rk.sL, -fk.l2s));
    const float rf = qf * ell;
    cs += (__builtin_fabsf(r) <= rk.tau) ? 0.0f : rf + qf;
    ck += rf - __builtin_amdgcn_fmed3f(rf, -rk.tau, rk.tau);
  }
}

// Returns x through an empty asm statement: the compiler must treat the result
// as a new value, so offsets derived from it are recomputed in each phase of
// a row instead of being kept (in registers or scratch) across phases.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Explicit waits on this wave's outstanding memory operations.  They are also
// compiler barriers: direct-to-LDS loads are not tracked by the compiler, so
// every LDS read of such data sits behind one of these.
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vmem_but() {  // all but the N most recent
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// All but the n most recent (n wave-uniform; counts above N wait as for N).
template <int N>
__device__ __forceinline__ void wait_vmem_upto(int n) {
  if constexpr (N == 0) {
    wait_vmem_all();
  } else {
    if (n >= N) wait_vmem_but<N>();
    else wait_vmem_upto<N - 1>(n);
  }
}

// Direct loads of slot s of a row's zp and zq into LDS slot position l.
template <int VAR, int AUX>
__device__ __forceinline__ void dma_slot(const RowIO<VAR>& io, Rsrc rzp, Rsrc rzq,
                                         typename Tr<VAR>::S (*lp)[kRowBlock],
                                         typename Tr<VAR>::S (*lq)[kRowBlock], int l, int s, int nvec,
                                         int tid) {
  if (io.has(io.nb(s, nvec))) {
    const uint32_t so = (uint32_t)s * RowIO<VAR>::SIN;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rzp, (__attribute__((address_space(3))) void*)&lp[l][io.wid * 64], 16, (uint32_t)tid * 16u, so, 0, AUX);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rzq, (__attribute__((address_space(3))) void*)&lq[l][io.wid * 64], 16, (uint32_t)tid * 16u, so, 0, AUX);
  }
}

// ---------------------------------------------------------------------------
// split rows: what the two halves of a verified row hand each other
// ---------------------------------------------------------------------------

// First-sweep statistics of a row or of one half (every lane holds the same
// values): max of zp and sum exp(s (zp - mp)) relative to it, the same of zq
// with K = sum exp(s (zq - mq)) (zq - zp), zq at the first index of mp, and
// (tempered form) sum exp(zq - mq).
struct XRec {
  float mp, sp, mq, sq, kq, za, sq1;
  int bi;
};

// Word i of a half's record, for lanes 0..n-1 (the others get 0): lane i
// publishes or reads word i.
__device__ __forceinline__ uint64_t* xrec(const FwdArgs& a, int row, int h) {
  return cold_args()->xres + ((long long)row * kMaxParts + h) * kXWords;
}

// Publishes n words (lane i: word i) of this half's record and returns, in
// lane i, word i of the partner's, once it carries this launch's tag
// (bounded wait; on expiry the launch reports AV_DEV_TIMEOUT).  Called by
// every wave with the same values; the last wave publishes.
__device__ __forceinline__ uint32_t xswap(const FwdArgs& a, uint64_t* mine, uint64_t* theirs, uint32_t v,
                                          int n, uint32_t tag) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == kLastWave && lane < n) tput(mine + lane, tag, v);
  uint64_t w = 0;
  Waiter wt(a.ctl, cold_args()->timeout_ticks);
  for (;;) {
    bool ok = true;
    if (lane < n) {
      w = tget(theirs + lane);
      ok = tag_ok(w, tag);
    }
    if (__all(ok)) break;
    if (!__all(wt.keep_going())) break;
  }
  return (uint32_t)w;
}

// Four parts: publishes n words (lane i < n: word i, at offset `off` of this
// part's record) and returns, in lane l < 4 n, word l % n of part l / n's
// record (this part's own words included), once each carries this launch's
// tag (bounded wait as above).  Called by every wave with the same values.
__device__ __forceinline__ uint32_t xgather4(const FwdArgs& a, int row, int ph, int off, uint32_t v, int n,
                                             uint32_t tag) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == kLastWave && lane < n) tput(xrec(a, row, ph) + off + lane, tag, v);
  const int o = lane / n, i = lane - o * n;
  const uint32_t own = (uint32_t)__shfl((int)v, i);
  const bool theirs = lane < n * 4 && o != ph;
  uint64_t w = 0;
  Waiter wt(a.ctl, cold_args()->timeout_ticks);
  for (;;) {
    bool ok = true;
    if (theirs) {
      w = tget(xrec(a, row, o) + off + i);
      ok = tag_ok(w, tag);
    }
    if (__all(ok)) break;
    if (!__all(wt.keep_going())) break;
  }
  return theirs ? (uint32_t)w : own;
}

// The statistics of the whole row from those of its halves, merged in a
// fixed order (first half, then second), so both partners get the same bits.
// The first half holds the lower indices: it wins ties of the maximum.
template <bool TM>
__device__ __forceinline__ XRec xmerge(const XRec& A, const XRec& B, float sL) {
  const float L = TM ? sL : kLog2e;
  XRec o;
  const bool second = B.mp > A.mp;
  o.bi = second ? B.bi : A.bi;
  o.za = second ? B.za : A.za;
  o.mp = fmaxf(A.mp, B.mp);
  const float fa = (A.sp == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((A.mp - o.mp) * L);
  const float fb = (B.sp == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((B.mp - o.mp) * L);
  o.sp = A.sp * fa + B.sp * fb;
  o.mq = fmaxf(A.mq, B.mq);
  const float ga = (A.sq == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((A.mq - o.mq) * L);
  const float gb = (B.sq == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((B.mq - o.mq) * L);
  o.sq = A.sq * ga + B.sq * gb;
  o.kq = A.kq * ga + B.kq * gb;
  o.sq1 = 0.0f;
  if constexpr (TM) {
    const float ha = (A.sq1 == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((A.mq - o.mq) * kLog2e);
    const float hb = (B.sq1 == 0.0f) ? 0.0f : __builtin_amdgcn_exp2f((B.mq - o.mq) * kLog2e);
    o.sq1 = A.sq1 * ha + B.sq1 * hb;
  }
  return o;
}

// The statistics of the whole row from those of its NP parts (2 or 4),
// merged in part order, so every part gets the same bits.
template <bool TM, int NP>
__device__ __forceinline__ XRec xchange_stats(const FwdArgs& a, const XRec& mine, int row, int ph,
                                              uint32_t tag, float sL) {
  const int lane = threadIdx.x & 63;
  uint32_t v = 0;
  switch (lane) {
    case 0: v = __float_as_uint(mine.mp); break;
    case 1: v = __float_as_uint(mine.sp); break;
    case 2: v = __float_as_uint(mine.mq); break;
    case 3: v = __float_as_uint(mine.sq); break;
    case 4: v = __float_as_uint(mine.kq); break;
    case 5: v = __float_as_uint(mine.za); break;
    case 6: v = __float_as_uint(mine.sq1); break;
    case 7: v = (uint32_t)mine.bi; break;
    default: break;
  }
  const uint32_t w = NP == 2 ? xswap(a, xrec(a, row, ph), xrec(a, row, ph ^ 1), v, 8, tag)
                             : xgather4(a, row, ph, 0, v, 8, tag);
  auto rec = [&](int o) {
    XRec r;
    r.mp = __uint_as_float(__shfl(w, 8 * o + 0));
    r.sp = __uint_as_float(__shfl(w, 8 * o + 1));
    r.mq = __uint_as_float(__shfl(w, 8 * o + 2));
    r.sq = __uint_as_float(__shfl(w, 8 * o + 3));
    r.kq = __uint_as_float(__shfl(w, 8 * o + 4));
    r.za = __uint_as_float(__shfl(w, 8 * o + 5));
    r.sq1 = __uint_as_float(__shfl(w, 8 * o + 6));
    r.bi = (int)__shfl(w, 8 * o + 7);
    return r;
  };
  if constexpr (NP == 2) {
    const XRec o = rec(0);  // the partner's
    return ph == 0 ? xmerge<TM>(mine, o, sL) : xmerge<TM>(o, mine, sL);
  } else {
    XRec m = rec(0);
    for (int o = 1; o < NP; ++o) m = xmerge<TM>(m, rec(o), sL);
    return m;
  }
}

// Clip corrections of the whole row: the parts' float64 values added in part
// order (the same bits in every part; for two parts either order gives them).
template <int NP>
__device__ __forceinline__ void xchange_clip(const FwdArgs& a, double& cs, double& ck, int row, int ph,
                                             uint32_t tag) {
  const int lane = threadIdx.x & 63;
  const uint64_t bs = (uint64_t)__double_as_longlong(cs), bk = (uint64_t)__double_as_longlong(ck);
  uint32_t v = 0;
  switch (lane) {
    case 0: v = (uint32_t)(bs >> 32); break;
    case 1: v = (uint32_t)bs; break;
    case 2: v = (uint32_t)(bk >> 32); break;
    case 3: v = (uint32_t)bk; break;
    default: break;
  }
  if constexpr (NP == 2) {
    const uint32_t w = xswap(a, xrec(a, row, ph) + 8, xrec(a, row, ph ^ 1) + 8, v, 4, tag);
    const uint64_t os = ((uint64_t)__shfl(w, 0) << 32) | (uint64_t)__shfl(w, 1);
    const uint64_t ok = ((uint64_t)__shfl(w, 2) << 32) | (uint64_t)__shfl(w, 3);
    cs = cs + __longlong_as_double((long long)os);
    ck = ck + __longlong_as_double((long long)ok);
  } else {
    const uint32_t w = xgather4(a, row, ph, 8, v, 4, tag);
    double ts = 0.0, tk = 0.0;
    for (int o = 0; o < NP; ++o) {
      const uint64_t os = ((uint64_t)__shfl(w, 4 * o + 0) << 32) | (uint64_t)__shfl(w, 4 * o + 1);
      const uint64_t ok = ((uint64_t)__shfl(w, 4 * o + 2) << 32) | (uint64_t)__shfl(w, 4 * o + 3);
      ts = o == 0 ? __longlong_as_double((long long)os) : ts + __longlong_as_double((long long)os);
      tk = o == 0 ? __longlong_as_double((long long)ok) : tk + __longlong_as_double((long long)ok);
    }
    cs = ts;
    ck = tk;
  }
}

// Verified row: statistics, loss, and (optionally) the gradient.
//
// Slots 0 .. nr-1 of the row stay in registers, nr .. nr+nl-1 in LDS, the
// rest are streamed (and read again for the gradient).  FULL: nr and nl are
// the compile-time maxima and the row fills every on-chip slot (the common
// case of a large vocabulary), so no on-chip access needs a guard.
//
// Split rows (SP = 2): the workgroup takes half ph of the row (vectors
// [0, pv0) or [pv0, nvec)) and its partner the other half, each on its own
// CU; the halves hand each other their first-sweep statistics and then their
// clip corrections, so both continue with the statistics of the whole row.
// SP = 4: the same with four parts of the row (boundaries on 64-vector
// multiples near the quarters), for launches with very few rows.
template <int VAR, bool FULL, bool GB, bool TM, int NRT, int SP>
__device__ __forceinline__ void verified_row(const FwdArgs& a, RowSmem& sm,
                                             typename Tr<VAR>::S (*lp)[kRowBlock],
                                             typename Tr<VAR>::S (*lq)[kRowBlock], const Item& it,
                                             int par, uint32_t tag, int ph) {
  using T = Tr<VAR>;
  using S = typename T::S;
  using IO = RowIO<VAR>;
  constexpr int NR = NRT, NL = RowCfg<VAR>::NL;
  constexpr uint32_t SIN = IO::SIN;
  int tid = opaque(threadIdx.x);
  const int lane = tid & 63, wid = tid >> 6;
  const int row = it.row;
  int vbase = 0, nvec = opaque_s(a.nvec);  // first vector and vectors of this part
  if constexpr (SP == 2) {
    const int pv0 = opaque_s(a.pv0);
    vbase = ph ? pv0 : 0;
    nvec = ph ? nvec - pv0 : pv0;
  } else if constexpr (SP == 4) {
    const long long N = nvec;
    auto bnd = [&](int i) {
      const long long b = ((N * i + 3) / 4 + 63) & ~63LL;
      return (int)(b < N ? b : N);
    };
    vbase = bnd(ph);
    nvec = (ph == 3 ? (int)N : bnd(ph + 1)) - vbase;
  }
  const int ebase = vbase * IO::VEC;              // row index of the part's first entry
  const long long rowv = (long long)row * a.nvec + vbase;
  const uint32_t rbytes = (uint32_t)nvec * (uint32_t)(IO::VEC * T::EB);
  const Rsrc rzp = row_rsrc(T::row(a.zp, rowv), rbytes);
  const Rsrc rzq = row_rsrc(T::row(a.zq, rowv), rbytes);
  const int nr = FULL ? NR : opaque_s(a.nr), nl = FULL ? NL : opaque_s(a.nl);
  const int von = nr + nl;             // first streamed slot
  const int nfull = nvec / kRowBlock;  // slots in which every thread has a vector
  const bool tail = nfull >= von;      // the partial slot nfull (if any) is streamed
  const float tau = opaque_s(a.tau);
  const float sL = TM ? opaque_s(a.inv_tl) : kLog2e;
  // lazy-rescale gaps of the tempered sums (see acc_vec): T kLazyGap, and at
  // most kLazyGap for the unscaled sum
  const float gp = TM ? kLazyGap * kLog2e / sL : kLazyGap, gq = fminf(gp, kLazyGap);

  // ---- sweep 1: read the row once; keep its on-chip slots, fold every
  // vector into the running statistics.  Fast form: the register slots and
  // then the streamed slots pass through the LDS slots two at a time (direct
  // loads, no registers held while in flight), then the LDS slots take their
  // resident data. ----
  constexpr bool RING = FULL && NL > 0;
  const int ns = nfull + (nfull * kRowBlock < nvec ? 1 : 0);  // slots, the partial one included
  if constexpr (!RING && NL > 0) {
    const IO io(tid, ebase);
#pragma unroll
    for (int l = 0; l < NL; ++l)
      if (l < nl) dma_slot<VAR, kAuxOnce>(io, rzp, rzq, lp, lq, l, nr + l, nvec, tid);
  }
  // Defined in every lane (zero where unused), so the register copies never
  // carry values from one row to the next.
  S rp[NR], rq[NR];
  {
    const IO io(tid, ebase);
#pragma unroll
    for (int v = 0; v < NR; ++v) {
      rp[v] = S{};
      rq[v] = S{};
      const int nbv = io.nb(v, nvec);
      if (!RING && v < nr && io.has(nbv)) {
        rp[v] = io.template load<kAuxOnce>(rzp, v, nbv);
        rq[v] = io.template load<kAuxOnce>(rzq, v, nbv);
      }
    }
  }
  RowAcc A;
  acc_init(A);
  if constexpr (RING) {
    // Every slot of the row comes in through the two halves of the LDS
    // slots, two slots at a time, double-buffered: the register slots first
    // (each copied from the LDS into its registers, then folded in), then
    // the streamed slots; each half then takes its resident slots.  Only
    // loads into the LDS are in flight, so every wait is counted here and the
    // first slots are folded in while the rest of the row is on its way.  A
    // wait for pair q leaves outstanding only what was issued after it (pair
    // q + 1, or a half's resident slots), counted for slots every wave loads.
    static_assert(NL == 4, "two halves of two LDS slots");
    constexpr int QR = (NR + 1) / 2;  // pairs that hold register slots
    const IO io(opaque(tid), ebase);
    const int nst = ns - von;              // streamed slots
    const int npair = (NR + nst + 1) >> 1;  // >= QR
    auto slot_of = [&](int e) { return e < NR ? e : von + (e - NR); };  // ring entry -> row slot
    const int nfullv = opaque(64);  // vectors of a wave block in a register slot
    auto ops_of = [&](int q) {  // loads of pair q that every wave issues (resident slots past the end)
      if (q >= npair) return 4;
      int n = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 2 * q + j;
        if (e < NR) n += 2;
        else if (e < NR + nst && von + (e - NR) < nfull) n += 2;
      }
      return n;
    };
    auto issue = [&](int q, int h) {  // pair q into half h, or the half's resident slots
      if (q < npair) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = 2 * q + j;
          if (e < NR) dma_slot<VAR, kAuxOnce>(io, rzp, rzq, lp, lq, 2 * h + j, e, nvec, tid);
          else if (e < NR + nst) dma_slot<VAR, kAuxFirst>(io, rzp, rzq, lp, lq, 2 * h + j, slot_of(e), nvec, tid);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) dma_slot<VAR, kAuxOnce>(io, rzp, rzq, lp, lq, 2 * h + j, nr + 2 * h + j, nvec, tid);
      }
    };
    auto wait_pair = [&](int q) {
      const int after = ops_of(q + 1);
      if (after >= 4) wait_vmem_but<4>();
      else if (after >= 2) wait_vmem_but<2>();
      else wait_vmem_all();
    };
    issue(0, 0);
    issue(1, 1);
#pragma unroll
    for (int q = 0; q < QR; ++q) {  // pairs with register slots (compile-time indices)
      const int h = q & 1;
      wait_pair(q);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 2 * q + j;
        if (e < NR) {
          if (io.has(nfullv)) {  // always: keeps one branch per register slot, as in the other forms
            rp[e] = io.lds(lp[2 * h + j], 64);
            rq[e] = io.lds(lq[2 * h + j], 64);
            acc_vec<VAR, TM>(rp[e], rq[e], io.lo(e), io.H(64), A, true, sL, gp, gq);
          }
        } else if (e < NR + nst) {
          const int sl = slot_of(e), nbv = io.nb(sl, nvec);
          if (io.has(nbv))
            acc_vec<VAR, TM>(io.lds(lp[2 * h + j], nbv), io.lds(lq[2 * h + j], nbv), io.lo(sl), io.H(nbv), A,
                             false, sL, gp, gq);
        }
      }
      wait_lds_reads();  // this half is free again
      issue(q + 2, h);
    }
    for (int q = QR; q < npair; ++q) {  // streamed pairs
      const int h = q & 1;
      wait_pair(q);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 2 * q + j;
        if (e < NR + nst) {
          const int sl = slot_of(e), nbv = io.nb(sl, nvec);
          if (io.has(nbv))
            acc_vec<VAR, TM>(io.lds(lp[2 * h + j], nbv), io.lds(lq[2 * h + j], nbv), io.lo(sl), io.H(nbv), A,
                             false, sL, gp, gq);
        }
      }
      wait_lds_reads();
      issue(q + 2, h);
    }
  } else {
    const IO io(opaque(tid), ebase);
#ifndef AV_SU
#define AV_SU 1
#endif
#pragma unroll AV_SU
    for (int s = von; s < nfull; ++s) {
      const S xp = io.template load<kAuxFirst>(rzp, s, 64), xq = io.template load<kAuxFirst>(rzq, s, 64);
      acc_vec<VAR, TM>(xp, xq, io.lo(s), io.H(64), A, false, sL, gp, gq);
    }
    if (tail) {
      const int nbv = io.nb(nfull, nvec);
      if (io.has(nbv)) {
        const S xp = io.template load<kAuxFirst>(rzp, nfull, nbv), xq = io.template load<kAuxFirst>(rzq, nfull, nbv);
        acc_vec<VAR, TM>(xp, xq, io.lo(nfull), io.H(nbv), A, false, sL, gp, gq);
      }
    }
  }
  uint64_t nxt = 0;
  if (tid == 0) nxt = claim(a);  // its reply returns behind this row's loads
  if constexpr (!RING) {  // the fast form folded its register slots in the ring
    const IO io(opaque(tid), ebase);
#pragma unroll
    for (int v = 0; v < NR; ++v) {
      const int nbv = io.nb(v, nvec);
      if (v < nr && io.has(nbv))
        acc_vec<VAR, TM>(rp[v], rq[v], io.lo(v), io.H(nbv), A, true, sL, gp, gq);
    }
  }
  if constexpr (NL > 0) {
    wait_vmem_all();  // the LDS copies of this wave have landed
    const IO io(opaque(tid), ebase);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int sl = nr + l, nbv = io.nb(sl, nvec);
      if (l < nl && io.has(nbv))
        acc_vec<VAR, TM>(io.lds(lp[l], nbv), io.lds(lq[l], nbv), io.lo(sl), io.H(nbv), A, true, sL, gp, gq);
    }
  }

  // ---- combine the statistics of the 1024 threads: row reductions inside
  // each wave, then every wave merges the 16 wave partials the same way ----
  RowAcc W = A;
  {  // the combine takes the zp sum relative to the running max
    const float L = TM ? sL : kLog2e;
    W.sp = (W.sp == 0.0f) ? 0.0f : W.sp * __builtin_amdgcn_exp2f((W.rp - W.mp) * L);
    W.rp = W.mp;
    wave_combine<TM>(W, L);
  }
  if (lane == 0) {
    sm.f[par][wid][0] = W.mp;
    sm.f[par][wid][1] = W.sp;
    sm.f[par][wid][2] = W.mq;
    sm.f[par][wid][3] = W.sq;
    sm.f[par][wid][4] = W.kq;
    sm.f[par][wid][5] = W.za;
    if constexpr (TM) sm.f1[par][wid] = W.sq1;
    sm.i[par][wid] = W.bi;
  }
  if (tid == 0) sm.item[par ^ 1] = nxt;
  __syncthreads();
  acc_init(W);
  if (lane < kRowWaves) {
    W.mp = sm.f[par][lane][0];
    W.sp = sm.f[par][lane][1];
    W.mq = sm.f[par][lane][2];
    W.sq = sm.f[par][lane][3];
    W.kq = sm.f[par][lane][4];
    W.za = sm.f[par][lane][5];
    if constexpr (TM) W.sq1 = sm.f1[par][lane];
    W.bi = sm.i[par][lane];
  }
  wave_combine<TM, 16>(W, TM ? sL : kLog2e);  // the 16 wave partials sit in lanes 0-15
  // (the tempered form keeps them in vector registers: through scalar
  // registers it measured slower, 0.8-1.2% at T = 0.5 and 2)
  XRec xr;
  if constexpr (TM) {
    xr = XRec{__shfl(W.mp, 0), __shfl(W.sp, 0), __shfl(W.mq, 0), __shfl(W.sq, 0), __shfl(W.kq, 0),
              __shfl(W.za, 0), __shfl(W.sq1, 0), __shfl(W.bi, 0)};
  } else {
    xr = XRec{bcast0(W.mp), bcast0(W.sp), bcast0(W.mq), bcast0(W.sq), bcast0(W.kq), bcast0(W.za), 0.0f,
              bcast0(W.bi)};
  }
  if constexpr (SP == 2 || SP == 4) xr = xchange_stats<TM, SP>(a, xr, row, ph, tag, sL);
  const float mp = xr.mp, sp = xr.sp;
  const float mq = xr.mq, sq = xr.sq, kq = xr.kq;
  const float zqa = xr.za;
  const int Arg = xr.bi;
  const float st = TM ? opaque_s(a.inv_t) : 1.0f;
  const float lse_p32 = TM ? __builtin_fmaf(mp, st, kLn2 * __builtin_amdgcn_logf(sp))
                           : mp + kLn2 * __builtin_amdgcn_logf(sp);
  const float lse_q32 = TM ? __builtin_fmaf(mq, st, kLn2 * __builtin_amdgcn_logf(sq))
                           : mq + kLn2 * __builtin_amdgcn_logf(sq);
  const float lse_q1 = TM ? mq + kLn2 * __builtin_amdgcn_logf(xr.sq1) : lse_q32;
  // sum_j q_j (log q_j - log p_j) = s sum_j q_j (zq_j - zp_j) - (lse_q - lse_p)
  const double KL = (double)st * ((double)kq / (double)sq) - (double)(lse_q32 - lse_p32);
  const RowK rk = row_consts<TM>(lse_p32, lse_q32, tau, st, sL);
  const FineK fk{mq, __builtin_amdgcn_logf(sq)};

  // ---- clipping: an entry's |r_j| = q_j |ell_j| is at most
  //   exp(m_t - lse_q) exp(zq_j - m_t) |zq_j - zp_j| + exp(zq_j - lse_q) |lse_q - lse_p|
  // (m_t: the thread's max zq).  Every entry of a region whose bound stays
  // below kClipCertify * tau lies inside the clip interval; only regions that
  // fail it are evaluated entry by entry, and S and the clipped KL follow from
  // the unclipped sums minus those corrections (zero for every entry inside
  // the interval, so a certified region would contribute nothing) ----
  // (tempered: exp(s m_t - lse_q) exp(s (zq_j - m_t)) s |zq_j - zp_j| + exp(s zq_j - lse_q) |delta|)
  const float adelta = __builtin_fabsf(rk.delta);
  bool flag_on, flag_st;
  if constexpr (TM) {
    const float ets = __builtin_amdgcn_exp2f(__builtin_fmaf(A.mq, sL, -rk.lseqL)) * st;
    flag_on = __builtin_fmaf(ets, A.pm_on,
                             adelta * __builtin_amdgcn_exp2f(__builtin_fmaf(A.mq_on, sL, -rk.lseqL))) >
              kClipCertify * tau;
    flag_st = __builtin_fmaf(ets, A.pm_st,
                             adelta * __builtin_amdgcn_exp2f(__builtin_fmaf(A.mq_st, sL, -rk.lseqL))) >
              kClipCertify * tau;
  } else {
    const float et = __builtin_amdgcn_exp2f((A.mq - lse_q32) * kLog2e);
    flag_on =
        __builtin_fmaf(et, A.pm_on, adelta * __builtin_amdgcn_exp2f((A.mq_on - lse_q32) * kLog2e)) >
        kClipCertify * tau;
    flag_st =
        __builtin_fmaf(et, A.pm_st, adelta * __builtin_amdgcn_exp2f((A.mq_st - lse_q32) * kLog2e)) >
        kClipCertify * tau;
  }
  float cs = 0.0f, ck = 0.0f;
  if (flag_on) {
    const IO io(opaque(tid), ebase);
#pragma unroll
    for (int v = 0; v < NR; ++v) {
      if (v < nr && io.has(io.nb(v, nvec)))
        clip_vec<VAR, TM, TM>(rp[v], rq[v], rk, fk, cs, ck);
    }
    if constexpr (NL > 0) {
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const int nbv = io.nb(nr + l, nvec);
        if (l < nl && io.has(nbv))
          clip_vec<VAR, TM, TM>(io.lds(lp[l], nbv), io.lds(lq[l], nbv), rk, fk, cs, ck);
      }
    }
  }
  if (flag_st) {
    const IO io(opaque(tid), ebase);
    for (int s = von; s < nfull; ++s) clip_vec<VAR, TM>(io.load(rzp, s, 64), io.load(rzq, s, 64), rk, fk, cs, ck);
    if (tail) {
      const int nbv = io.nb(nfull, nvec);
      if (io.has(nbv)) clip_vec<VAR, TM>(io.load(rzp, nfull, nbv), io.load(rzq, nfull, nbv), rk, fk, cs, ck);
    }
  }
  double dcs = 0.0, dck = 0.0;
  if (__any(flag_on || flag_st)) {
    dcs = xsum<64>((double)cs);
    dck = xsum<64>((double)ck);
  }
  if (lane == 0) {
    sm.d[par][wid][0] = dcs;
    sm.d[par][wid][1] = dck;
  }
  __syncthreads();
  // (no wave with a correction: every partial is zero, and so are the sums)
  const double pcs = (lane < kRowWaves) ? sm.d[par][lane][0] : 0.0;
  const double pck = (lane < kRowWaves) ? sm.d[par][lane][1] : 0.0;
  double tcs = 0.0, tck = 0.0;
  if (__any(pcs != 0.0 || pck != 0.0)) {
    tcs = wsumd16(pcs);
    tck = wsumd16(pck);
  }
  if constexpr (SP == 2 || SP == 4) {
    if (tau < INFINITY) xchange_clip<SP>(a, tcs, tck, row, ph, tag);  // with tau = inf all are 0
  }
  const double S64 = (KL + 1.0) - tcs, KLc64 = KL - tck;
  const float S32 = (float)S64;

  // ---- the row is complete: one wave publishes it (split rows: the first
  // half's); if it is the request's last verified row to complete, that wave
  // also finishes the request ----
  if ((SP == 1 || ph == 0) && wid == kLastWave) {
    uint32_t n = 0;
    if (lane == 0) {
      const KArgs K = cold_args();
      const double ce = (double)lse_q1 - (double)zqa;
      const double lam = (double)opaque_s(a.lam);
      const float loss = (float)(lam * ce + (1.0 - lam) * KLc64);
      K->row_loss[row] = loss;
      K->tgt[row] = Arg;
      if (K->stats)
        store16(K->stats + 4 * (long long)row, (f32x4){lse_p32, lse_q32, S32, (float)KLc64});
      if (K->lse1) K->lse1[row] = lse_q1;
      tput(K->rowres + 2 * (long long)row, tag, (uint32_t)Arg);
      tput(K->rowres + 2 * (long long)row + 1, tag, __float_as_uint(loss));
      n = arrive(K->arrive + it.req, tag);
    }
    n = bcast0(n);
    if (n == (uint32_t)it.bkb) finish_request(a, it.req, it.r0, it.bkb, tag);
  }

  // ---- sweep 2: the gradient; streamed vectors are read a second time
  // (fast form: through the LDS slots once their resident data is done) ----
  if (a.grad) {
    const GradK gk = grad_consts<TM>(opaque_s(a.lam), opaque_s(a.gs), S32, st, lse_q1, rk.delta);
    const Rsrc rg = grad_rsrc<GB, IO::VEC>(a.grad, rowv, nvec * IO::VEC);
    if constexpr (RING) {
      // Each LDS half's resident slots' gradient frees the half; the streamed
      // slots then come in again two at a time, double-buffered, the first
      // two pairs behind the register slots' gradient.  A wait for pair q
      // leaves outstanding what was issued after it (half 1's resident and
      // the register slots' stores, pair q - 1's stores, pair q + 1's loads),
      // counted where every wave issues them, so the stores in flight need
      // not drain.
      constexpr int SPS = IO::kHalves ? 2 : 1;  // stores of one vector's gradient
      constexpr int kRegStores = NR * SPS;      // all register slots are full
      static_assert(kRegStores + 4 * SPS + 4 <= 63, "vmcnt range");
      static_assert(NL == 4, "two halves of two LDS slots");
      const IO io(opaque(tid), ebase);
      const int np2 = (ns - von + 1) >> 1;
      auto full = [&](int q, int j) { return q < np2 && von + 2 * q + j < nfull; };
      auto loads_of = [&](int q) { return (full(q, 0) ? 2 : 0) + (full(q, 1) ? 2 : 0); };
      auto stores_of = [&](int q) { return (full(q, 0) ? SPS : 0) + (full(q, 1) ? SPS : 0); };
      auto reread = [&](int q, int h) {
        if (q < np2) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int sl = von + 2 * q + j;
            if (sl < ns) dma_slot<VAR, kAuxAgain>(io, rzp, rzq, lp, lq, 2 * h + j, sl, nvec, tid);
          }
        }
      };
      // Each half's resident slots, then its first streamed pair.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          grad_vec<VAR, GB, TM>(io.lds(lp[2 * h + j], 64), io.lds(lq[2 * h + j], 64), io, nr + 2 * h + j, 64, rk,
                                gk, Arg, rg, flag_on);
        wait_lds_reads();
        reread(h, h);
      }
#pragma unroll
      for (int v = 0; v < NR; ++v) grad_vec<VAR, GB, TM>(rp[v], rq[v], io, v, 64, rk, gk, Arg, rg, flag_on);
      for (int q = 0; q < np2; ++q) {
        const int h = q & 1;
        const int after = q == 0   ? 2 * SPS + loads_of(1) + kRegStores
                          : q == 1 ? kRegStores + stores_of(0) + loads_of(2)
                                   : stores_of(q - 1) + loads_of(q + 1);
        wait_vmem_upto<kRegStores + 4 * SPS + 4>(after);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int sl = von + 2 * q + j;
          if (sl < ns) {
            const int nbv = io.nb(sl, nvec);
            if (io.has(nbv))
              grad_vec<VAR, GB, TM>(io.lds(lp[2 * h + j], nbv), io.lds(lq[2 * h + j], nbv), io, sl, nbv, rk, gk,
                                    Arg, rg, flag_st);
          }
        }
        wait_lds_reads();  // this half is free again
        reread(q + 2, h);
      }
      wait_lds_reads();  // the next row's direct loads may overwrite the LDS slots
    } else {
      {
        const IO io(opaque(tid), ebase);
#ifndef AV_GU
#define AV_GU 2
#endif
#pragma unroll AV_GU
        for (int s = von; s < nfull; ++s) {
          const S xp = io.template load<kAuxAgain>(rzp, s, 64), xq = io.template load<kAuxAgain>(rzq, s, 64);
          grad_vec<VAR, GB, TM>(xp, xq, io, s, 64, rk, gk, Arg, rg, flag_st);
        }
        if (tail) {
          const int nbv = io.nb(nfull, nvec);
          if (io.has(nbv)) {
            const S xp = io.template load<kAuxAgain>(rzp, nfull, nbv), xq = io.template load<kAuxAgain>(rzq, nfull, nbv);
            grad_vec<VAR, GB, TM>(xp, xq, io, nfull, nbv, rk, gk, Arg, rg, flag_st);
          }
        }
      }
      {
        const IO io(opaque(tid), ebase);
#pragma unroll
        for (int v = 0; v < NR; ++v) {
          const int nbv = io.nb(v, nvec);
          if (v < nr && io.has(nbv))
            grad_vec<VAR, GB, TM>(rp[v], rq[v], io, v, nbv, rk, gk, Arg, rg, flag_on);
        }
      }
      if constexpr (NL > 0) {
        const IO io(opaque(tid), ebase);
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          const int sl = nr + l, nbv = io.nb(sl, nvec);
          if (l < nl && io.has(nbv))
            grad_vec<VAR, GB, TM>(io.lds(lp[l], nbv), io.lds(lq[l], nbv), io, sl, nbv, rk, gk, Arg, rg, flag_on);
        }
      }
      wait_lds_reads();
    }
  }
}

// SP = 2: split rows.  Workgroups 2p and 2p+1 form pair p and take the
// pair's rows in a fixed order (items p, p + pairs, ...): workgroup 2p + h
// takes half h of each (unverified rows as the two halves of their argmax
// scan).  Both halves of a verified row are therefore in progress together,
// and a half only waits for its partner, which works through the same list.
// SP = 3: a split tail (ragged layout, every row verified).  Items 0 ..
// nwhole-1 are whole rows; then each remaining row is two consecutive items,
// its halves.  Items are claimed from the dispenser in order, and every
// workgroup of the launch is resident, so the partner of a claimed half is
// either claimed already (and in progress) or the next item that any
// workgroup claims when it finishes its current one: no half waits on a
// half that cannot start.  The halves use kPairRegs register slots in the
// fast form (FULL), the row's slot counts otherwise.
template <int VAR, bool FULL, bool GB, bool TM, int NRT, int SP>
__global__ __launch_bounds__(kRowBlock) void fused_kernel(FwdArgs a) {
  using S = typename Tr<VAR>::S;
  constexpr int NLA = RowCfg<VAR>::NL > 0 ? RowCfg<VAR>::NL : 1;
  __shared__ S lp[NLA][kRowBlock];
  __shared__ S lq[NLA][kRowBlock];
  __shared__ RowSmem sm;
  // ragged: row offsets [B + 1]; dense longest-first: b_k [B] (uint8, padded
  // to 8 bytes), then order [B] (uint16)
  extern __shared__ int s_dyn[];
  const int* s_off = s_dyn;
  uint8_t* key = (uint8_t*)s_dyn;
  uint16_t* order = (uint16_t*)(key + (a.lpt ? (a.B + 7) & ~7 : 0));
  const int tid = threadIdx.x;
  if (tid == 0) {
    // both requests in flight at once (the launch boundary already orders
    // this launch after the previous one's writes)
    const uint32_t epoch =
        (uint32_t)__hip_atomic_load(a.ctl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.item[0] = claim(a);  // split rows: only its status bits are used
    sm.tag = epoch + 1u;  // epochs stay below 0xFFFFFFFF, so tags are never 0
  }
  int bad = 0;
  if (a.ragged) {
    for (int j = tid; j <= a.B; j += kRowBlock) s_dyn[j] = a.row_off[j];
    __syncthreads();
    int okl = 1;
    for (int j = tid; j < a.B; j += kRowBlock) {
      const int n = s_off[j + 1] - s_off[j];
      if (n < 1 || n > a.k) okl = 0;
    }
    if (tid == 0 && (s_off[0] != 0 || s_off[a.B] != a.R)) okl = 0;
    bad = !__syncthreads_and(okl);
    if (bad && tid == 0) raise_status(a.ctl, AV_DEV_BAD_OFFSETS);
  } else if (a.lpt) {  // counting sort of the requests by b_k, descending
    if (tid <= a.k) sm.hist[tid] = 0;
    if (tid < 8) key[((a.B + 7) & ~7) - 1 - tid] = 0;  // padding (no b_k is 0)
    __syncthreads();
    for (int b = tid; b < a.B; b += kRowBlock) {
      const int kb = min(max(a.bk[b], 1), a.k);
      key[b] = (uint8_t)kb;
      atomicAdd(&sm.hist[kb], 1);
    }
    __syncthreads();
    if (tid <= a.k) {
      int c = 0;
      for (int v = tid + 1; v <= a.k; ++v) c += sm.hist[v];
      sm.cnt[tid] = c;
    }
    __syncthreads();
    if (tid == 0) {
      int cv = 0, cu = 0;
      for (int p = 0; p <= a.k; ++p) {
        sm.cum[p] = cv;
        sm.cumu[p] = cu;
        if (p < a.k) {
          cv += sm.cnt[p];
          cu += a.B - sm.cnt[p];
        }
      }
    }
    for (int b = tid; b < a.B; b += kRowBlock) {  // stable: rank among equal b_k
      const int kb = key[b];
      // requests j < b with the same b_k, eight keys per LDS read: a byte of
      // x is 0 exactly where key[j] == kb
      const uint64_t* k8 = (const uint64_t*)key;
      const uint64_t pat = 0x0101010101010101ull * (uint64_t)kb;
      int rank = 0;
      for (int q = 0; q < (b >> 3); ++q) rank += zero_bytes(k8[q] ^ pat);
      if (b & 7) {  // bytes of the last word at j >= b count as different
        const uint64_t keep = (1ull << (8 * (b & 7))) - 1ull;
        rank += zero_bytes((k8[b >> 3] ^ pat) | ~keep);
      }
      order[sm.cnt[kb] + rank] = (uint16_t)b;
    }
  }
  __syncthreads();
  const uint32_t tag = sm.tag;
  // Work items: rows, with the unverified rows of the longest-first order
  // counted twice (two halves each) unless rows are split (a pair takes both
  // halves of each of its rows).
  // (unverified rows in quarters count four times: the last nq of them)
  const int nq = SP == 1 && a.lpt ? min(a.nquart, a.R - sm.cum[a.k]) : 0;
  const uint32_t nitems =
      SP == 3 ? (uint32_t)(2 * a.R - a.nwhole)
              : (uint32_t)a.R + (SP == 1 && a.lpt ? (uint32_t)(a.R - sm.cum[a.k] + 2 * nq) : 0u);
  // split rows: teams of SP consecutive workgroups, one part of a row each
  constexpr int NPT = SP == 4 ? 4 : 2;
  constexpr bool TEAM = SP == 2 || SP == 4;
  const int ph = TEAM ? (int)(blockIdx.x % NPT) : 0;
  const uint32_t pair = blockIdx.x / NPT, npairs = gridDim.x / NPT;
  for (int iter = 0;; ++iter) {
    const int par = iter & 1;
    const uint64_t w = sm.item[par];
    const uint32_t idx = TEAM ? pair + (uint32_t)iter * npairs : __builtin_amdgcn_readfirstlane((uint32_t)w);
    const uint32_t stat = __builtin_amdgcn_readfirstlane((uint32_t)(w >> 32));
    if (idx >= nitems) break;
    if (bad || stat != 0u) {  // failed launch: drain without work
      if (tid == 0) sm.item[par ^ 1] = claim(a);
      __syncthreads();
      continue;
    }
    if constexpr (SP == 3) {
      const int h = (int)idx - a.nwhole;
      if (h >= 0) {
        const Item it = map_item(a, sm, s_off, order, key, a.nwhole + (h >> 1), false);
        verified_row<VAR, FULL, GB, TM, FULL ? kPairRegs : NRT, 2>(a, sm, lp, lq, it, par, tag, h & 1);
        continue;
      }
    }
    Item it = map_item(a, sm, s_off, order, key, (int)idx, TEAM, nq);
    if (TEAM && !it.verified) {
      it.half = ph;
      it.nparts = NPT;
    }
    if (it.verified) verified_row<VAR, FULL, GB, TM, NRT, SP == 3 ? 1 : SP>(a, sm, lp, lq, it, par, tag, ph);
    else unverified_row<VAR, GB>(a, sm, it.row, par, it.half, it.nparts, tag);
  }
  // The workgroup that leaves last sums the request losses, reports the
  // status, resets the dispenser and the done count, and advances the epoch.
  // Status bits and the done count share one word, so every status raised
  // before a workgroup left is seen by the one that leaves last.
  __syncthreads();
  if (tid == 0)
    sm.exitw = __hip_atomic_fetch_add(a.ctl + 2, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint64_t old = sm.exitw;
  if ((uint32_t)old == gridDim.x - 1u) {
    uint32_t stat = (uint32_t)(old >> 32) | (bad ? (uint32_t)AV_DEV_BAD_OFFSETS : 0u);
    if (stat == 0u && !finish_total(a, sm, tag)) stat |= (uint32_t)AV_DEV_TIMEOUT;
    if (tid == 0) {
      const KArgs K = cold_args();
      if (K->status_out) K->status_out[0] = (int32_t)stat;
      __hip_atomic_store(a.ctl, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ctl + 2, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t epoch = tag - 1u;
      const uint32_t next = (epoch + 1u == 0xFFFFFFFFu) ? 0u : epoch + 1u;
      __hip_atomic_store(a.ctl + 1, (uint64_t)next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// standalone backward
// ---------------------------------------------------------------------------

template <int VAR, bool GB, bool TM>
__global__ __launch_bounds__(kBlock) void bwd_kernel(BwdArgs a) {
  using T = Tr<VAR>;
  using S = typename T::S;
  constexpr int VEC = T::VEC, NVMAX = T::NVMAX;
  const int tid = threadIdx.x;
  const uint32_t item = blockIdx.x;
  const int row = (int)(item / (uint32_t)a.C);
  const int chunk = (int)(item - (uint32_t)row * (uint32_t)a.C);
  bool verified = true;
  if (!a.ragged) {
    const int req = row / a.k, pos = row - req * a.k;
    verified = pos < min(max(a.bk[req], 1), a.k);
  }
  const long long rowv = (long long)row * a.nvec;
  const int vlo = (int)((uint32_t)chunk * (uint32_t)a.nvec / (uint32_t)a.C);
  const int vhi = (int)((uint32_t)(chunk + 1) * (uint32_t)a.nvec / (uint32_t)a.C);
  const void* zp_r = T::row(a.zp, rowv);
  const void* zq_r = T::row(a.zq, rowv);
  float* g_r = (float*)a.grad + rowv * VEC;
  uint16_t* gb_r = (uint16_t*)a.grad + rowv * VEC;
  // bfloat16 rows (8 entries per vector): each wave takes a block of 64
  // vectors, and lane l the entries 4l..4l+3 of the block's first half and
  // the same four of its second half (halves of 4 nbv entries), so every
  // store instruction of a wave writes one contiguous stretch (with 8
  // consecutive entries per lane each 16-byte store would fill only half of
  // every 32 bytes, and the gradient's write traffic would nearly double).
  constexpr bool kHalves = VAR == kBf16x8;
  const int lane = tid & 63, wid = tid >> 6;
  auto block_of = [&](int v, int& base, int& nbv) {
    base = vlo + v * kBlock + wid * 64;
    nbv = min(max(vhi - base, 0), 64);
  };
  if (!verified) {
    float z[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) z[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      if constexpr (kHalves) {
        int base, nbv;
        block_of(v, base, nbv);
        if (lane < nbv) {
          const long long e0 = 8LL * base + 4 * lane, e1 = e0 + 4LL * nbv;
          if constexpr (GB) {
            __builtin_nontemporal_store((u32x2){0u, 0u}, (u32x2*)(gb_r + e0));
            __builtin_nontemporal_store((u32x2){0u, 0u}, (u32x2*)(gb_r + e1));
          } else {
            store16_nt(g_r + e0, (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
            store16_nt(g_r + e1, (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
          }
        }
      } else {
        const int vi = vlo + v * kBlock + tid;
        if (vi < vhi) {
          if constexpr (GB) store_vec_bf16<VEC>(gb_r, (unsigned)vi, z);
          else store_vec<VEC>(g_r, (unsigned)vi, z);
        }
      }
    }
    return;
  }
  const f32x4 st = *(const f32x4*)(a.stats + 4 * (long long)row);
  const int A = a.tgt[row];
  const RowK rk = row_consts<TM>(st[0], st[1], a.tau, a.inv_t, a.inv_tl);
  const GradK gk = grad_consts<TM>(a.lam, a.gs, st[2], a.inv_t, TM ? a.lse1[row] : 0.0f, rk.delta);
  S xp[NVMAX], xq[NVMAX];
  if constexpr (kHalves) {
    const char* pb = (const char*)zp_r;
    const char* qb = (const char*)zq_r;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      int base, nbv;
      block_of(v, base, nbv);
      if (lane < nbv) {
        const long long o0 = 16LL * base + 8 * lane, o1 = o0 + 8LL * nbv;
        const u32x2 p0 = *(const u32x2*)(pb + o0), p1 = *(const u32x2*)(pb + o1);
        const u32x2 q0 = *(const u32x2*)(qb + o0), q1 = *(const u32x2*)(qb + o1);
        xp[v] = S{p0.x, p0.y, p1.x, p1.y};
        xq[v] = S{q0.x, q0.y, q1.x, q1.y};
      }
    }
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      int base, nbv;
      block_of(v, base, nbv);
      if (lane < nbv) {
        const long long e0 = 8LL * base + 4 * lane, e1 = e0 + 4LL * nbv;
        float out[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float q, ell, r;
          opd_entry<TM>(T::at(xp[v], e), T::at(xq[v], e), rk, q, ell, r);
          out[e] = grad_entry<TM>(q, T::at(xq[v], e) - T::at(xp[v], e), r, T::at(xq[v], e), rk.tau, gk);
          if ((e < 4 ? e0 + e : e1 + (e - 4)) == (long long)A) out[e] = out[e] - gk.fix;
        }
        if constexpr (GB) {
          __builtin_nontemporal_store((u32x2){pack_bf16(out[0], out[1]), pack_bf16(out[2], out[3])},
                                      (u32x2*)(gb_r + e0));
          __builtin_nontemporal_store((u32x2){pack_bf16(out[4], out[5]), pack_bf16(out[6], out[7])},
                                      (u32x2*)(gb_r + e1));
        } else {
          store16_nt(g_r + e0, (f32x4){out[0], out[1], out[2], out[3]});
          store16_nt(g_r + e1, (f32x4){out[4], out[5], out[6], out[7]});
        }
      }
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
      xp[v] = T::load(zp_r, (unsigned)vi);
      xq[v] = T::load(zq_r, (unsigned)vi);
    }
  }
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float q, ell, r;
        opd_entry<TM>(T::at(xp[v], e), T::at(xq[v], e), rk, q, ell, r);
        out[e] = grad_entry<TM>(q, T::at(xq[v], e) - T::at(xp[v], e), r, T::at(xq[v], e), rk.tau, gk);
        if (vi * VEC + e == A) out[e] = out[e] - gk.fix;
      }
      if constexpr (GB) store_vec_bf16<VEC>(gb_r, (unsigned)vi, out);
      else store_vec<VEC>(g_r, (unsigned)vi, out);
    }
  }
}

// ---------------------------------------------------------------------------
// length head and workspace fill
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// length head: prediction, and its online update
// ---------------------------------------------------------------------------

// sigmoid(w . h_b + bias) in float64 for the workgroup's request: per-thread
// partial dot products, wave butterflies, then the wave partials in a fixed
// order (the same bits on every call).  Every thread gets the result.
__device__ __forceinline__ double head_rate(const float* hb, const float* w, int H, double bias,
                                            double* s) {
  const int tid = threadIdx.x;
  double acc = 0.0;
  if (H % 4 == 0 && ((uintptr_t)hb % 16u) == 0 && ((uintptr_t)w % 16u) == 0) {
    // 16-byte loads, four per operand in flight before the fp64 FMAs
    const f32x4* h4 = (const f32x4*)hb;
    const f32x4* w4 = (const f32x4*)w;
    const int n4 = H >> 2;
    int j = tid;
    for (; j + 3 * kBlock < n4; j += 4 * kBlock) {
      f32x4 x[4], y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = h4[j + u * kBlock];
        y[u] = w4[j + u * kBlock];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fma((double)x[u][e], (double)y[u][e], acc);
    }
    for (; j < n4; j += kBlock) {
      const f32x4 x = h4[j], y = w4[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fma((double)x[e], (double)y[e], acc);
    }
  } else {
    for (int j = tid; j < H; j += kBlock) acc = fma((double)hb[j], (double)w[j], acc);
  }
  acc = wsumd(acc);
  if ((tid & 63) == 0) s[tid >> 6] = acc;
  __syncthreads();
  const double z = ((s[0] + s[1]) + (s[2] + s[3])) + bias;
  if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
  const double e = exp(z);
  return e / (1.0 + e);
}

__global__ __launch_bounds__(kBlock) void head_kernel(HeadArgs a) {
  __shared__ double s[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const double sg = head_rate(a.h + (long long)b * a.H, a.w, a.H, (double)a.bias, s);
  if (tid == 0) {
    const double x = (double)a.gamma * sg * (double)a.k;
    const double n = a.mode == 0 ? ceil(x) : floor(x);
    const int bk = n < 1.0 ? 1 : (n > (double)a.k ? a.k : (int)n);
    a.bk[b] = bk;
    if (a.rate) a.rate[b] = (float)sg;
  }
}

// Online update, step 1 (one workgroup per request): the prediction, the
// label acc_b / b_k, and d loss / d z_b = 2 (rate_b - label_b) rate_b (1 - rate_b) / B
// with loss = mean_b (rate_b - label_b)^2.  ws[b] = d loss / d z_b,
// ws[B + b] = (rate_b - label_b)^2.
__global__ __launch_bounds__(kBlock) void head_grad_kernel(HeadUpdArgs a) {
  __shared__ double s[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const double sg = head_rate(a.h + (long long)b * a.H, a.w, a.H, (double)a.bias[0], s);
  if (tid == 0) {
    const int n = min(max(a.bk[b], 1), a.k);
    const double e = sg - (double)a.acc[b] / (double)n;
    a.ws[b] = 2.0 * e * sg * (1.0 - sg) / (double)a.B;
    a.ws[a.B + b] = e * e;
    if (a.rate) a.rate[b] = (float)sg;
  }
}

// One AdamW step on one parameter held in float32 (arithmetic in float64):
// decoupled weight decay, then bias-corrected moments.  th0, m0, v0: the
// values before the step.
__device__ __forceinline__ void adamw_from(float* th, float* m, float* v, float th0, float m0, float v0, double g,
                                          const HeadUpdArgs& a) {
  const double mm = a.beta1 * (double)m0 + (1.0 - a.beta1) * g;
  const double vv = a.beta2 * (double)v0 + (1.0 - a.beta2) * g * g;
  double t = (double)th0 * (1.0 - a.lr * a.wd);
  t -= (a.lr / a.bc1) * mm / (sqrt(vv) / a.sqrt_bc2 + a.eps);
  *th = (float)t;
  *m = (float)mm;
  *v = (float)vv;
}

// Online update, step 2: workgroup g owns weights 64 g .. 64 g + 63 (lane =
// weight) and its 8 waves split the requests (wave w takes b = w, w + 8, ...).
// g_w[j] = sum_b dz_b h[b, j]: each wave sums its requests in order, then the
// 8 wave sums are added in wave order; d loss / d h[b, j] = dz_b w[j] (the
// weight before the step); then wave 0 takes the AdamW step on its weights.
// Wave 0 of workgroup 0 also sums g_bias and the loss (per lane in request
// order, then lanes by a fixed butterfly) and steps the bias.
constexpr int kStepWaves = 8, kStepCols = 64, kStepChunk = 1024;

// Workgroup barrier for LDS data only: global stores still in flight are not
// waited for (nothing in the workgroup reads them back).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kStepWaves * 64) void head_step_kernel(HeadUpdArgs a) {
  constexpr int kG = 16;  // requests of a wave whose loads go out together
  __shared__ double part[kStepWaves][kStepCols];
  __shared__ double sdz[kStepChunk];
  __shared__ double ssq[kStepChunk];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int j = blockIdx.x * kStepCols + lane;
  const bool in = j < a.H;
  const bool bias_wg = blockIdx.x == 0;
  // Everything the step reads is requested up front (the weight, its moments,
  // the bias state, the first group of h values) and every value is taken
  // into registers before the first store of d loss / d h: a wait for a load
  // issued before a store also waits for that store.
  float w0 = 0.0f, m0 = 0.0f, v0 = 0.0f, b0v = 0.0f, mb = 0.0f, vb = 0.0f;
  if (in) {
    w0 = a.w[j];
    m0 = a.m_w[j];
    v0 = a.v_w[j];
  }
  if (bias_wg && tid == 0) {
    b0v = a.bias[0];
    mb = a.m_b[0];
    vb = a.v_b[0];
  }
  const double wj = (double)w0;
  double g = 0.0, gb = 0.0, sq = 0.0;
  for (int b0 = 0; b0 < a.B; b0 += kStepChunk) {
    const int nb = min(kStepChunk, a.B - b0);
    const float* hj = a.h + (long long)b0 * a.H + j;
    float x[kG];
    auto load_group = [&](int i0) {
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int i = i0 + u * kStepWaves;
        x[u] = (in && i < nb) ? hj[(long long)i * a.H] : 0.0f;
      }
    };
    load_group(wid);
    if (b0 > 0) lds_barrier();  // the previous chunk's readers are done
    for (int i = tid; i < nb; i += kStepWaves * 64) {
      sdz[i] = a.ws[b0 + i];
      if (bias_wg) ssq[i] = a.ws[a.B + b0 + i];
    }
    lds_barrier();
    for (int i0 = wid; i0 < nb; i0 += kG * kStepWaves) {
      if (i0 != wid) load_group(i0);
      double d[kG];
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int i = i0 + u * kStepWaves;
        d[u] = i < nb ? sdz[i] : 0.0;
        if (i < nb) g = fma(d[u], (double)x[u], g);
      }
      asm volatile("" : "+v"(m0), "+v"(v0), "+v"(b0v), "+v"(mb), "+v"(vb));
      if (in && a.grad_h) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          const int i = i0 + u * kStepWaves;
          if (i < nb) a.grad_h[(long long)(b0 + i) * a.H + j] = (float)(d[u] * wj);
        }
      }
    }
    // workgroup 0, wave 0: g_bias and the squared errors, per lane in
    // request order
    if (bias_wg && wid == 0) {
      for (int i = lane; i < nb; i += 64) {
        gb += sdz[i];
        sq += ssq[i];
      }
    }
  }
  part[wid][lane] = g;
  lds_barrier();
  if (wid == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kStepWaves; ++w) t += part[w][lane];
    if (in) adamw_from(a.w + j, a.m_w + j, a.v_w + j, w0, m0, v0, t, a);
    if (bias_wg) {
      gb = wsumd(gb);
      sq = wsumd(sq);
      if (lane == 0) {
        if (a.loss) a.loss[0] = (float)(sq / (double)a.B);
        adamw_from(a.bias, a.m_b, a.v_b, b0v, mb, vb, gb, a);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// sampling-based verification
//
// Position i of a block is accepted with probability min(1, p_i(d_i) /
// q_i(d_i)) up to the first rejection; the token that replaces the first
// rejected draft is drawn from max(0, p - q) by an exponential race:
// argmax_j r_j / E_j with E_j = -ln u_j, u_j from Philox4x32-10 keyed by the
// caller's seed at counter (j / 4, row, 0, 0), word j % 4.
// ---------------------------------------------------------------------------

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC 2011): each round
// multiplies words 0 and 2 by the round constants and mixes the high and low
// halves of the products with words 1 and 3 and the key, which is bumped by
// the Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd > 0) {
      k0 += W0;
      k1 += W1;
    }
    // full 64-bit products: one multiply instruction gives both halves
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

// E = -ln(u), u = (w + 1/2) / 2^32, to about 1e-7 relative.  Where u is
// within 1/16 of 1, u itself would lose the low bits of 1 - u in float32, so
// E comes from v = 1 - u = (2^32 - 1 - w + 1/2) / 2^32 by the series
// -ln(1 - v) = v (1 + v/2 + v^2/3 + ...) (7 terms: the tail is below
// (1/16)^7); elsewhere from the hardware log2 of u.
__device__ __forceinline__ float race_exponential(uint32_t w) {
  constexpr float k2m32 = 0x1p-32f;
  const float v = ((float)(0xFFFFFFFFu - w) + 0.5f) * k2m32;
  if (v < 0.0625f) {
    float t = 1.0f / 7.0f;
    t = __builtin_fmaf(t, v, 1.0f / 6.0f);
    t = __builtin_fmaf(t, v, 0.2f);
    t = __builtin_fmaf(t, v, 0.25f);
    t = __builtin_fmaf(t, v, 1.0f / 3.0f);
    t = __builtin_fmaf(t, v, 0.5f);
    t = __builtin_fmaf(t, v, 1.0f);
    return v * t;
  }
  return -kLn2 * __builtin_amdgcn_logf(((float)w + 0.5f) * k2m32);
}

// Per-thread online (max, sum exp) of zp and zq over a row.
struct SpecAcc {
  float mp, sp, mq, sq;
};

template <int VAR>
__device__ __forceinline__ void spec_fold(const typename Tr<VAR>::S& xp, const typename Tr<VAR>::S& xq,
                                          SpecAcc& A) {
  using T = Tr<VAR>;
  float vp = T::at(xp, 0), vq = T::at(xq, 0);
#pragma unroll
  for (int e = 1; e < T::VEC; ++e) {
    vp = fmaxf(vp, T::at(xp, e));
    vq = fmaxf(vq, T::at(xq, e));
  }
  const float np = fmaxf(A.mp, vp), nq = fmaxf(A.mq, vq);
  A.sp *= __builtin_amdgcn_exp2f((A.mp - np) * kLog2e);
  A.sq *= __builtin_amdgcn_exp2f((A.mq - nq) * kLog2e);
  A.mp = np;
  A.mq = nq;
  const float npL = np * kLog2e, nqL = nq * kLog2e;
#pragma unroll
  for (int e = 0; e < T::VEC; ++e) {
    A.sp += __builtin_amdgcn_exp2f(__builtin_fmaf(T::at(xp, e), kLog2e, -npL));
    A.sq += __builtin_amdgcn_exp2f(__builtin_fmaf(T::at(xq, e), kLog2e, -nqL));
  }
}

// Dense layout: the w-th verified row in request-major order, or -1 when
// there are fewer than w + 1 (one wave's prefix scan over the requests).
__device__ __forceinline__ int nth_verified_row(const SpecArgs& a, int w) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int nb = b < a.B ? min(max(a.bk[b], 1), a.k) : 0;
    int incl = nb;  // inclusive prefix sum over the lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int excl = base + incl - nb;
    const uint64_t hit = __ballot(nb > 0 && w >= excl && w < excl + nb);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      return __shfl((b0 + lane) * a.k + (w - excl), src);
    }
    base += __shfl(incl, 63);
  }
  return -1;
}

// Step 1, one 256-thread workgroup per verified row: lse_p, lse_q and the
// acceptance decision u * q(d) < p(d) (a draft outside [0, V) is rejected).
// In the dense layout workgroup w takes the w-th verified row (the launch has
// one per stored row; the surplus exit), so consecutive workgroups, which the
// dispatcher spreads over the CUs, hold rows at every position and the
// verified rows spread evenly.
template <int VAR>
__global__ __launch_bounds__(kBlock) void spec_stats_kernel(SpecArgs a) {
  using T = Tr<VAR>;
  using S = typename T::S;
  constexpr uint32_t VB = T::VEC * T::EB;
  __shared__ float s[kWaves][4];
  __shared__ int s_row;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (blockIdx.x == 0 && tid == 0 && a.status) a.status[0] = 0;
  int r = blockIdx.x;
  if (!a.ragged) {
    if (wid == 0) {
      const int row = nth_verified_row(a, (int)blockIdx.x);
      if (lane == 0) s_row = row;
    }
    __syncthreads();
    r = s_row;
    if (r < 0) return;
  }
  const long long rowv = (long long)r * a.nvec;
  const Rsrc rzp = row_rsrc(T::row(a.zp, rowv), (uint32_t)a.V * T::EB);
  const Rsrc rzq = row_rsrc(T::row(a.zq, rowv), (uint32_t)a.V * T::EB);
  SpecAcc A = {-INFINITY, 0.0f, -INFINITY, 0.0f};
  int v = tid;
  for (; v + 3 * kBlock < a.nvec; v += 4 * kBlock) {
    S xp[4], xq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xp[j] = T::template bload<kAuxOnce>(rzp, (uint32_t)(v + j * kBlock) * VB, 0);
      xq[j] = T::template bload<kAuxOnce>(rzq, (uint32_t)(v + j * kBlock) * VB, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) spec_fold<VAR>(xp[j], xq[j], A);
  }
  for (; v < a.nvec; v += kBlock)
    spec_fold<VAR>(T::template bload<kAuxOnce>(rzp, (uint32_t)v * VB, 0),
                   T::template bload<kAuxOnce>(rzq, (uint32_t)v * VB, 0), A);
  // combine: butterflies (empty threads have s = 0), then the 4 waves in order
  float dummy = 0.0f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float omp = __shfl_xor(A.mp, o), osp = __shfl_xor(A.sp, o);
    const float omq = __shfl_xor(A.mq, o), osq = __shfl_xor(A.sq, o);
    lse_merge(A.mp, A.sp, dummy, omp, osp, 0.0f);
    lse_merge(A.mq, A.sq, dummy, omq, osq, 0.0f);
  }
  if (lane == 0) {
    s[wid][0] = A.mp;
    s[wid][1] = A.sp;
    s[wid][2] = A.mq;
    s[wid][3] = A.sq;
  }
  __syncthreads();
  if (tid == 0) {
    SpecAcc G = {s[0][0], s[0][1], s[0][2], s[0][3]};
    for (int w = 1; w < kWaves; ++w) {
      lse_merge(G.mp, G.sp, dummy, s[w][0], s[w][1], 0.0f);
      lse_merge(G.mq, G.sq, dummy, s[w][2], s[w][3], 0.0f);
    }
    const float lse_p = G.mp + kLn2 * __builtin_amdgcn_logf(G.sp);
    const float lse_q = G.mq + kLn2 * __builtin_amdgcn_logf(G.sq);
    const int d = a.draft[r];
    uint32_t acc = 0u;
    if ((unsigned)d < (unsigned)a.V) {
      const float pd = __builtin_amdgcn_exp2f((T::elem(T::row(a.zp, rowv), d) - lse_p) * kLog2e);
      const float qd = __builtin_amdgcn_exp2f((T::elem(T::row(a.zq, rowv), d) - lse_q) * kLog2e);
      acc = (a.u[r] * qd < pd) ? 1u : 0u;
    }
    const u32x4 rec = {acc, __float_as_uint(lse_p), __float_as_uint(lse_q), 0u};
    *(u32x4*)(a.ws + 4 * (long long)r) = rec;  // one 16-byte record per row
    settle16(rec);
    if (a.stats) {
      a.stats[2 * (long long)r] = lse_p;
      a.stats[2 * (long long)r + 1] = lse_q;
    }
  }
}

// Step 1 with the row statistics given (the fused pass computed lse_p and
// lse_q of every verified row in its first sweep): one thread per stored row
// gathers p(d) and q(d) and takes the acceptance test; no row is read whole.
template <int VAR>
__global__ __launch_bounds__(kBlock) void spec_gather_kernel(SpecArgs a) {
  using T = Tr<VAR>;
  const long long r = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (r == 0 && a.status) a.status[0] = 0;
  if (r >= a.R) return;
  if (!a.ragged) {
    const int b = (int)(r / a.k), i = (int)(r - (long long)b * a.k);
    if (i >= min(max(a.bk[b], 1), a.k)) return;  // not verified
  }
  const float lse_p = a.stats_in[r * a.stats_stride], lse_q = a.stats_in[r * a.stats_stride + 1];
  const long long rowv = r * a.nvec;
  const int d = a.draft[r];
  uint32_t acc = 0u;
  if ((unsigned)d < (unsigned)a.V) {
    const float pd = __builtin_amdgcn_exp2f((T::elem(T::row(a.zp, rowv), d) - lse_p) * kLog2e);
    const float qd = __builtin_amdgcn_exp2f((T::elem(T::row(a.zq, rowv), d) - lse_q) * kLog2e);
    acc = (a.u[r] * qd < pd) ? 1u : 0u;
  }
  const u32x4 rec = {acc, __float_as_uint(lse_p), __float_as_uint(lse_q), 0u};
  *(u32x4*)(a.ws + 4 * r) = rec;
  settle16(rec);
  if (a.stats) {
    a.stats[2 * r] = lse_p;
    a.stats[2 * r + 1] = lse_q;
  }
}

// Race keys of one entry: r_j / E_j with r_j = max(0, p_j - q_j), and p_j / E_j
// (the draw from p, used when the residual is zero everywhere).  Keeps the
// largest of each, lowest index on ties.
struct RaceBest {
  float rk, pk;
  int ri, pi;
};
__device__ __forceinline__ void race_keep(float key, int j, float& best, int& bi) {
  if (key > best || (key == best && j < bi)) {
    best = key;
    bi = j;
  }
}
__device__ __forceinline__ void race_entry(float zpj, float zqj, uint32_t w, int j, float lpL, float lqL,
                                           RaceBest& R) {
  const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zpj, kLog2e, -lpL));
  const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(zqj, kLog2e, -lqL));
  const float ie = __builtin_amdgcn_rcpf(race_exponential(w));
  race_keep(fmaxf(p - q, 0.0f) * ie, j, R.rk, R.ri);
  race_keep(p * ie, j, R.pk, R.pi);
}
__device__ __forceinline__ void race_merge(RaceBest& R, const RaceBest& O) {
  race_keep(O.rk, O.ri, R.rk, R.ri);
  race_keep(O.pk, O.pi, R.pk, R.pi);
}
// The wave's best residual and p draws in every lane: DPP steps inside each
// row of 16 lanes, then the four rows in order (a selection under a total
// order, so the result is the same whatever the pairing; all lanes active).
template <int C>
__device__ __forceinline__ void race_step(RaceBest& R) {
  const RaceBest O{dpp<C>(R.rk), dpp<C>(R.pk), dpp<C>(R.ri), dpp<C>(R.pi)};
  race_merge(R, O);
}
__device__ __forceinline__ void race_wave(RaceBest& R) {
  race_step<kDppSwap1>(R);
  race_step<kDppSwap2>(R);
  race_step<kDppMirror8>(R);
  race_step<kDppMirror16>(R);
  RaceBest B{lane_of(R.rk, 0), lane_of(R.pk, 0), lane_of(R.ri, 0), lane_of(R.pi, 0)};
#pragma unroll
  for (int r = 1; r < 4; ++r)
    race_merge(B, RaceBest{lane_of(R.rk, 16 * r), lane_of(R.pk, 16 * r), lane_of(R.ri, 16 * r),
                           lane_of(R.pi, 16 * r)});
  R = B;
}

// The accepted length of request b: the first verified position whose test
// failed (n if none).  Run by one wave; every lane gets the result.
__device__ __forceinline__ int spec_first(const SpecArgs& a, int r0, int n) {
  const int lane = threadIdx.x & 63;
  const bool rej = lane < n && a.ws[4 * (long long)(r0 + lane)] == 0u;
  const uint64_t m = __ballot(rej);
  return m ? (__ffsll((unsigned long long)m) - 1) : n;
}

// Request b's rows (r0, n); false if its ragged offsets are invalid.
__device__ __forceinline__ bool spec_span(const SpecArgs& a, int b, int& r0, int& n) {
  if (a.ragged) {
    r0 = a.row_off[b];
    n = a.row_off[b + 1] - r0;
    return n >= 1 && n <= a.k && r0 >= 0 && r0 + n <= a.R;
  }
  r0 = b * a.k;
  n = min(max(a.bk[b], 1), a.k);
  return true;
}

// Step 2, workgroup (c, b): chunk c of the row at request b's first
// rejection (vectors [c C, (c+1) C), C = a.chunk): the chunk's best race keys
// -> chunk record [b][c] = {residual key, its index, p key, its index}.
template <int VAR>
__global__ __launch_bounds__(kBlock) void spec_race_kernel(SpecArgs a) {
  using T = Tr<VAR>;
  using S = typename T::S;
  constexpr int VEC = T::VEC;
  constexpr uint32_t VB = VEC * T::EB;
  __shared__ RaceBest s_r[kWaves];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int r0, n;
  if (!spec_span(a, b, r0, n)) return;
  __shared__ int s_first;
  if (wid == 0) {
    const int f = spec_first(a, r0, n);
    if (lane == 0) s_first = f;
  }
  __syncthreads();
  const int first = s_first;
  if (first >= n) return;
  const int row = r0 + first;
  const uint32_t* wsr = a.ws + 4 * (long long)row;
  const float lpL = __uint_as_float(wsr[1]) * kLog2e, lqL = __uint_as_float(wsr[2]) * kLog2e;
  const long long rowv = (long long)row * a.nvec;
  const Rsrc rzp = row_rsrc(T::row(a.zp, rowv), (uint32_t)a.V * T::EB);
  const Rsrc rzq = row_rsrc(T::row(a.zq, rowv), (uint32_t)a.V * T::EB);
  const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
  RaceBest R = {-1.0f, -1.0f, INT_MAX, INT_MAX};
  const int v1 = min((c + 1) * a.chunk, a.nvec);
  for (int v = c * a.chunk + tid; v < v1; v += kBlock) {
    const S xp = T::template bload<kAuxOnce>(rzp, (uint32_t)v * VB, 0);
    const S xq = T::template bload<kAuxOnce>(rzq, (uint32_t)v * VB, 0);
    const int j0 = v * VEC;
#pragma unroll
    for (int g = 0; g < (VEC + 3) / 4; ++g) {  // one generator call per 4 entries
      uint32_t c0 = (uint32_t)(j0 + 4 * g) >> 2, c1 = (uint32_t)row, c2 = 0u, c3 = 0u;
      philox4x32_10(c0, c1, c2, c3, k0, k1);
      const uint32_t wd[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int e = 0; e < (VEC < 4 ? VEC : 4); ++e) {
        const int ee = 4 * g + e, j = j0 + ee;
        race_entry(T::at(xp, ee), T::at(xq, ee), wd[j & 3], j, lpL, lqL, R);
      }
    }
  }
  race_wave(R);
  if (lane == 0) s_r[wid] = R;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) race_merge(R, s_r[w]);
    const u32x4 rec = {__float_as_uint(R.rk), (uint32_t)R.ri, __float_as_uint(R.pk), (uint32_t)R.pi};
    *(u32x4*)(a.chunks + 4 * ((long long)b * a.nchunk + c)) = rec;
    settle16(rec);
  }
}

// Step 3, one wave per request: the accepted length, and the token from the
// chunk records (chunk order; the residual's draw unless every residual key
// is zero, then p's).
__global__ __launch_bounds__(64) void spec_finish_kernel(SpecArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int r0, n;
  if (!spec_span(a, b, r0, n)) {  // invalid ragged offsets: nothing is verified
    if (lane == 0) {
      a.acc[b] = 0;
      a.token[b] = -1;
      if (a.status) atomicOr(a.status, (int32_t)AV_DEV_BAD_OFFSETS);
    }
    return;
  }
  const int first = spec_first(a, r0, n);
  int token = -1;
  if (first < n) {
    RaceBest R = {-1.0f, -1.0f, INT_MAX, INT_MAX};
    if (lane < a.nchunk) {
      const uint32_t* rec = a.chunks + 4 * ((long long)b * a.nchunk + lane);
      R.rk = __uint_as_float(rec[0]);
      R.ri = (int)rec[1];
      R.pk = __uint_as_float(rec[2]);
      R.pi = (int)rec[3];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      RaceBest O;
      O.rk = __shfl_xor(R.rk, o);
      O.ri = __shfl_xor(R.ri, o);
      O.pk = __shfl_xor(R.pk, o);
      O.pi = __shfl_xor(R.pi, o);
      race_merge(R, O);
    }
    token = R.rk > 0.0f ? R.ri : R.pi;
  }
  if (lane == 0) {
    a.acc[b] = first;
    a.token[b] = token;
  }
}

__global__ __launch_bounds__(kBlock) void zero_kernel(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock)
    p[i] = 0ull;
}

// The kernel forms built: whole rows (every variant, general or fast form);
// split rows for the 16-byte variants, in the general form or in the fast
// form with kRowRegs16 or kPairRegs register slots; whole rows with a split
// tail for the 16-byte variants, general or fast; rows in four parts for the
// 16-byte variants, general form.
enum Form {
  kWholeGeneral, kWholeFast, kSplitGeneral, kSplitFast, kSplitFastPair, kTailGeneral, kTailFast, kQuartGeneral
};
inline Form form_of(bool full, int split, int nr) {
  if (split == 4) return kQuartGeneral;
  if (split == 3) return full ? kTailFast : kTailGeneral;
  if (split != 2) return full ? kWholeFast : kWholeGeneral;
  if (!full) return kSplitGeneral;
  return nr == kPairRegs ? kSplitFastPair : kSplitFast;
}
template <int VAR, bool GB, bool TM>
const void* kernel_of(Form f) {
  constexpr bool kWideVar = VAR == kBf16x8 || VAR == kF32x4;
  switch (f) {
    case kWholeFast: return (const void*)fused_kernel<VAR, true, GB, TM, RowCfg<VAR>::NR, 1>;
    case kWholeGeneral: return (const void*)fused_kernel<VAR, false, GB, TM, RowCfg<VAR>::NR, 1>;
    default: break;
  }
  if constexpr (kWideVar) {
    switch (f) {
      case kSplitGeneral: return (const void*)fused_kernel<VAR, false, GB, TM, kRowRegs16, 2>;
      case kSplitFast: return (const void*)fused_kernel<VAR, true, GB, TM, kRowRegs16, 2>;
      case kSplitFastPair: return (const void*)fused_kernel<VAR, true, GB, TM, kPairRegs, 2>;
      case kTailGeneral: return (const void*)fused_kernel<VAR, false, GB, TM, RowCfg<VAR>::NR, 3>;
      case kTailFast: return (const void*)fused_kernel<VAR, true, GB, TM, RowCfg<VAR>::NR, 3>;
      case kQuartGeneral: return (const void*)fused_kernel<VAR, false, GB, TM, kPairRegs, 4>;
      default: break;
    }
  }
  return nullptr;
}
template <int VAR>
const void* kernel_t(Form f, bool gb, bool tm) {
  if (tm) return gb ? kernel_of<VAR, true, true>(f) : kernel_of<VAR, false, true>(f);
  return gb ? kernel_of<VAR, true, false>(f) : kernel_of<VAR, false, false>(f);
}
const void* fused_kernel_ptr(Variant v, Form f, bool gb, bool tm) {
  switch (v) {
    case kBf16x8: return kernel_t<kBf16x8>(f, gb, tm);
    case kBf16x1: return kernel_t<kBf16x1>(f, gb, tm);
    case kF32x4: return kernel_t<kF32x4>(f, gb, tm);
    default: return kernel_t<kF32x1>(f, gb, tm);
  }
}
template <int VAR, bool TM>
hipError_t launch_bwd_g(const BwdArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.R * (unsigned)a.C;
  if (a.gbf16) hipLaunchKernelGGL((bwd_kernel<VAR, true, TM>), dim3(grid), dim3(kBlock), 0, s, a);
  else hipLaunchKernelGGL((bwd_kernel<VAR, false, TM>), dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}
template <int VAR>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  return a.tm ? launch_bwd_g<VAR, true>(a, s) : launch_bwd_g<VAR, false>(a, s);
}

}  // namespace

hipError_t launch_fused(Variant v, bool full, int nr, const FwdArgs& a, int grid, size_t lds, hipStream_t s) {
  const void* k = fused_kernel_ptr(v, form_of(full, a.split, nr), a.gbf16 != 0, a.tm != 0);
  if (!k) return hipErrorInvalidDeviceFunction;
  FwdArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(k, dim3(grid), dim3(kRowBlock), params, lds, s);
}

hipError_t fused_blocks_per_cu(Variant v, bool full, int split, int nr, bool gb, bool tm, size_t lds, int* out) {
  const void* k = fused_kernel_ptr(v, form_of(full, split, nr), gb, tm);
  if (!k) {
    *out = 0;
    return hipSuccess;
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, k, kRowBlock, lds);
}

hipError_t launch_bwd(Variant v, const BwdArgs& a, hipStream_t s) {
  switch (v) {
    case kBf16x8: return launch_bwd_t<kBf16x8>(a, s);
    case kBf16x1: return launch_bwd_t<kBf16x1>(a, s);
    case kF32x4: return launch_bwd_t<kF32x4>(a, s);
    default: return launch_bwd_t<kF32x1>(a, s);
  }
}

hipError_t launch_head(const HeadArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(head_kernel, dim3(a.B), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int VAR>
hipError_t launch_spec_t(const SpecArgs& a, hipStream_t s) {
  if (a.stats_in)
    hipLaunchKernelGGL(spec_gather_kernel<VAR>, dim3((unsigned)((a.R + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(spec_stats_kernel<VAR>, dim3(a.R), dim3(kBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_race_kernel<VAR>, dim3(a.nchunk, a.B), dim3(kBlock), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_finish_kernel, dim3(a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_spec(Variant v, const SpecArgs& a, hipStream_t s) {
  switch (v) {
    case kBf16x8: return launch_spec_t<kBf16x8>(a, s);
    case kBf16x1: return launch_spec_t<kBf16x1>(a, s);
    case kF32x4: return launch_spec_t<kF32x4>(a, s);
    default: return launch_spec_t<kF32x1>(a, s);
  }
}

hipError_t launch_head_update(const HeadUpdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(head_grad_kernel, dim3(a.B), dim3(kBlock), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_step_kernel, dim3((a.H + kStepCols - 1) / kStepCols), dim3(kStepWaves * 64), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_zero(uint64_t* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, words);
  return hipGetLastError();
}

}  // namespace avk
