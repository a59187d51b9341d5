// gfx950 kernels for the AdaFlash verify + on-policy-distillation pass.
//
// What is computed is defined in include/av.h (after the Pith review page of
// "AdaFlash: Adaptive Speculative Decoding via On-Policy Distilled Diffusion
// Drafters": "What carries the argument", Referee Report major comment 2 and
// minor comment 2, the free-parameter ledger).  This file is about how.
//
// fused_kernel -- the whole forward (+ gradient) pass in one launch.
//   A row's statistics (lse_p, lse_q, argmax, then the clipped-KL sum and S)
//   depend on the entire V-long row, and the gradient of every entry depends
//   on S.  Streaming a row twice from HBM would cost 12 bytes per verified
//   bf16 entry instead of 8 (4 read + 4 written), so a row is split into C
//   chunks that C workgroups hold in registers while they exchange per-chunk
//   partials, twice, through the workspace; every byte of zp/zq is read from
//   HBM exactly once and every gradient byte is written once.
//
//   Work items (row, chunk) are handed out in row-major order by an atomic
//   counter to a persistent grid.  Only running workgroups take items, and
//   every item before the one a workgroup waits on has already been taken,
//   so the lowest unfinished row always has all of its chunks held by
//   running workgroups: the waits cannot deadlock as long as C workgroups
//   fit on the device at once (C <= 64, far below one per CU).
//
//   Every exchanged value is one 64-bit word {tag, 32-bit payload} written
//   and read with agent-scope atomics, so each word is coherent across XCDs
//   on its own and no cache-wide fence is needed.  The tag is the launch
//   epoch (kept in the workspace, advanced by the last workgroup), so stale
//   words of earlier launches never match and nothing is cleared between
//   launches; graph replays see a fresh epoch too.
//
//   Each wait is bounded (wall clock); on expiry the launch raises
//   AV_DEV_TIMEOUT, every other wait gives up at once, and the grid drains.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ void raise_status(uint64_t* ctl, uint32_t bits) {
  __hip_atomic_fetch_or(ctl, (uint64_t)bits << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait: sleeps a little between polls, and every few polls gives
// up if the launch already failed or the wall-clock bound is exceeded.
struct Waiter {
  long long t0, limit;
  uint64_t* ctl;
  int it;
  __device__ Waiter(uint64_t* c, long long lim) : t0(wall_clock64()), limit(lim), ctl(c), it(0) {}
  __device__ bool keep_going() {
    if ((++it & 7) == 0) {
      if ((uint32_t)(tget(ctl) >> 32) != 0u) return false;
      if (wall_clock64() - t0 > limit) {
        raise_status(ctl, AV_DEV_TIMEOUT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
  }
};

// ---------------------------------------------------------------------------
// wave64 reductions (xor butterflies: every lane ends with the same bits)
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
__device__ __forceinline__ void wargmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    amax_merge(v, i, ov, oi);
  }
}

// ---------------------------------------------------------------------------
// element access per variant
// ---------------------------------------------------------------------------

template <int VAR>
struct Tr;

template <>
struct Tr<kBf16x8> {  // 8 bfloat16 per 16-byte load
  static constexpr int VEC = 8, NVMAX = 4;
  using S = u32x4;
  __device__ static S load(const void* base, long long vi) { return ((const u32x4*)base)[vi]; }
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
  static constexpr int VEC = 1, NVMAX = 16;
  using S = uint32_t;
  __device__ static S load(const void* base, long long vi) { return ((const uint16_t*)base)[vi]; }
  __device__ static float at(const S& s, int) { return __uint_as_float(s << 16); }
  __device__ static float elem(const void* base, long long j) {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[j] << 16);
  }
};

template <>
struct Tr<kF32x4> {  // 4 float32 per 16-byte load
  static constexpr int VEC = 4, NVMAX = 8;
  using S = f32x4;
  __device__ static S load(const void* base, long long vi) { return ((const f32x4*)base)[vi]; }
  __device__ static float at(const S& s, int e) { return s[e]; }
  __device__ static float elem(const void* base, long long j) { return ((const float*)base)[j]; }
};

template <>
struct Tr<kF32x1> {
  static constexpr int VEC = 1, NVMAX = 16;
  using S = float;
  __device__ static S load(const void* base, long long vi) { return ((const float*)base)[vi]; }
  __device__ static float at(const S& s, int) { return s; }
  __device__ static float elem(const void* base, long long j) { return ((const float*)base)[j]; }
};

template <int VEC>
__device__ __forceinline__ void store_vec(float* g, long long off, const float* v) {
  if constexpr (VEC == 8) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    const f32x4 b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, (f32x4*)(g + off));
    __builtin_nontemporal_store(b, (f32x4*)(g + off + 4));
  } else if constexpr (VEC == 4) {
    const f32x4 a = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(a, (f32x4*)(g + off));
  } else {
    __builtin_nontemporal_store(v[0], g + off);
  }
}

// ---------------------------------------------------------------------------
// per-entry math shared by the fused and the standalone backward pass
// ---------------------------------------------------------------------------

struct RowK {
  float lseqL, delta, tau;
};
__device__ __forceinline__ RowK row_consts(float lse_p, float lse_q, float tau) {
  RowK k;
  k.lseqL = lse_q * kLog2e;
  k.delta = lse_q - lse_p;
  k.tau = tau;
  return k;
}
// q_j = exp(zq_j - lse_q); r_j = q_j (log q_j - log p_j), with the log-ratio
// formed from the logits; g_j = c_j (r_j + q_j) = c_j q_j (ell_j + 1).
__device__ __forceinline__ void opd_entry(float zp, float zq, const RowK& k, float& q, float& r,
                                          float& g) {
  q = __builtin_amdgcn_exp2f(__builtin_fmaf(zq, kLog2e, -k.lseqL));
  const float ell = (zq - zp) - k.delta;
  r = q * ell;
  g = (__builtin_fabsf(r) <= k.tau) ? (r + q) : 0.0f;
}

// d loss / d zq_j = gs [lam (q_j - [j = a]) + (1 - lam)(g_j - S q_j)]
//                 = A q_j + Bc g_j - [j = a] gs lam
struct GradK {
  float a, b, fix;
};
__device__ __forceinline__ GradK grad_consts(float lam, float gs, float S) {
  GradK g;
  g.a = gs * (lam - (1.0f - lam) * S);
  g.b = gs * (1.0f - lam);
  g.fix = gs * lam;
  return g;
}
__device__ __forceinline__ float grad_entry(float q, float g, const GradK& c) {
  return __builtin_fmaf(c.a, q, c.b * g);
}

// ---------------------------------------------------------------------------
// fused pass
// ---------------------------------------------------------------------------

struct Smem {
  float f[kWaves][4];
  int i[kWaves];
  double d[kWaves];
  float rf[4];
  int ri;
  double rd[2];
  uint32_t item, stat, tag;
};

// Request `req` is complete once every one of its rows has published its
// result word; called by the workgroup that finished the request's last item.
__device__ __forceinline__ void finish_request(const FwdArgs& a, const int* s_off, int req,
                                            uint32_t tag) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) != 0) return;
  int r0, n, bkb;
  if (a.ragged) {
    r0 = s_off[req];
    n = s_off[req + 1] - r0;
    bkb = n;
  } else {
    r0 = req * a.k;
    n = a.k;
    bkb = min(max(a.bk[req], 1), a.k);
  }
  uint64_t w0 = 0, w1 = 0;
  Waiter wt(a.ctl, a.timeout_ticks);
  for (;;) {
    bool ok = true;
    if (lane < n) {
      w0 = tget(a.rowres + 2 * (long long)(r0 + lane));
      w1 = tget(a.rowres + 2 * (long long)(r0 + lane) + 1);
      ok = tag_ok(w0, tag) && tag_ok(w1, tag);
    }
    if (__all(ok)) break;
    if (!__all(wt.keep_going())) break;
  }
  const bool inb = lane < bkb;
  bool match = false;
  if (inb) match = a.draft[r0 + lane] == (int32_t)(uint32_t)w0;
  const uint64_t mism = __ballot(inb && !match);
  const int acc = mism ? (__ffsll((unsigned long long)mism) - 1) : bkb;
  double v = inb ? (double)lo_f(w1) : 0.0;
  v = wsumd(v);
  if (lane == 0) {
    a.acc[req] = acc;
    if (a.req_loss) a.req_loss[req] = (float)v;
    const uint64_t bits = (uint64_t)__double_as_longlong(v);
    tput(a.reqres + 2 * (long long)req, tag, (uint32_t)(bits >> 32));
    tput(a.reqres + 2 * (long long)req + 1, tag, (uint32_t)bits);
  }
}

// Sum of the request totals in a fixed order; run by the workgroup that
// holds the last item, after its own request has been finished.
__device__ __forceinline__ void finish_total(const FwdArgs& a, Smem& sm, uint32_t tag) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double part = 0.0;
  for (int b = tid; b < a.B; b += kBlock) {
    uint64_t h = 0, l = 0;
    Waiter wt(a.ctl, a.timeout_ticks);
    do {
      h = tget(a.reqres + 2 * (long long)b);
      l = tget(a.reqres + 2 * (long long)b + 1);
      if (tag_ok(h, tag) && tag_ok(l, tag)) break;
    } while (wt.keep_going());
    part += __longlong_as_double((long long)(((uint64_t)(uint32_t)h << 32) | (uint32_t)l));
  }
  part = wsumd(part);
  if (lane == 0) sm.d[wid] = part;
  __syncthreads();
  if (tid == 0 && a.total) a.total[0] = (float)((sm.d[0] + sm.d[1]) + (sm.d[2] + sm.d[3]));
}

template <int VAR>
__device__ __forceinline__ void process_item(const FwdArgs& a, Smem& sm, const int* s_off,
                                             uint32_t item, uint32_t tag) {
  using T = Tr<VAR>;
  using S = typename T::S;
  constexpr int VEC = T::VEC, NVMAX = T::NVMAX;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  const int row = (int)(item / (uint32_t)a.C);
  const int chunk = (int)(item - (uint32_t)row * (uint32_t)a.C);
  const bool owner = chunk == a.C - 1;  // publishes the row's result
  int req, pos, bkb;
  bool last_of_req;
  if (a.ragged) {
    int lo = 0, hi = a.B - 1;  // last request whose first row is <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= row) lo = mid;
      else hi = mid - 1;
    }
    req = lo;
    pos = row - s_off[req];
    bkb = s_off[req + 1] - s_off[req];
    last_of_req = owner && row == s_off[req + 1] - 1;
  } else {
    req = row / a.k;
    pos = row - req * a.k;
    bkb = min(max(a.bk[req], 1), a.k);
    last_of_req = owner && pos == a.k - 1;
  }
  const bool verified = pos < bkb;
  const long long rowv = (long long)row * a.nvec;
  const int vlo = (int)((long long)chunk * a.nvec / a.C);
  const int vhi = (int)((long long)(chunk + 1) * a.nvec / a.C);
  uint64_t* slot_row = a.slots + (long long)row * kMaxChunks * kSlotWords;
  uint64_t* my_slot = slot_row + chunk * kSlotWords;

  // ---- stream the chunk into registers (one HBM read of each byte) ----
  S xp[NVMAX], xq[NVMAX];
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
      xp[v] = T::load(a.zp, rowv + vi);
      if (verified) xq[v] = T::load(a.zq, rowv + vi);
    }
  }

  // ---- round 1, local: max + first argmax of zp, max of zq ----
  float mp = -INFINITY, mq = -INFINITY;
  int ip = INT_MAX;
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = T::at(xp[v], e);
        if (x > mp) {
          mp = x;
          ip = vi * VEC + e;
        }
      }
      if (verified) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) mq = fmaxf(mq, T::at(xq[v], e));
      }
    }
  }
  wargmax(mp, ip);
  mq = wmax(mq);
  if (lane == 0) {
    sm.f[wid][0] = mp;
    sm.i[wid] = ip;
    sm.f[wid][1] = mq;
  }
  __syncthreads();
  float Mp = sm.f[0][0], Mq = sm.f[0][1];
  int Ap = sm.i[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    amax_merge(Mp, Ap, sm.f[w][0], sm.i[w]);
    Mq = fmaxf(Mq, sm.f[w][1]);
  }

  if (!verified) {
    if (tid == 0) {
      tput(my_slot + 0, tag, __float_as_uint(Mp));
      tput(my_slot + 1, tag, (uint32_t)Ap);
    }
    if (a.grad) {
      float z[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) z[e] = 0.0f;
#pragma unroll
      for (int v = 0; v < NVMAX; ++v) {
        const int vi = vlo + v * kBlock + tid;
        if (vi < vhi) store_vec<VEC>(a.grad, (rowv + vi) * VEC, z);
      }
    }
    if (owner && wid == 0) {  // combine the row's argmax partials
      uint64_t w0 = 0, w1 = 0;
      Waiter wt(a.ctl, a.timeout_ticks);
      for (;;) {
        bool ok = true;
        if (lane < a.C) {
          w0 = tget(slot_row + lane * kSlotWords + 0);
          w1 = tget(slot_row + lane * kSlotWords + 1);
          ok = tag_ok(w0, tag) && tag_ok(w1, tag);
        }
        if (__all(ok)) break;
        if (!__all(wt.keep_going())) break;
      }
      float m = -INFINITY;
      int ix = INT_MAX;
      if (lane < a.C) {
        m = lo_f(w0);
        ix = (int)(uint32_t)w1;
      }
      wargmax(m, ix);
      if (lane == 0) {
        a.tgt[row] = ix;
        a.row_loss[row] = 0.0f;
        if (a.stats) *(f32x4*)(a.stats + 4 * (long long)row) = (f32x4){0.f, 0.f, 0.f, 0.f};
        tput(a.rowres + 2 * (long long)row, tag, (uint32_t)ix);
        tput(a.rowres + 2 * (long long)row + 1, tag, 0u);
      }
    }
  } else {
    // ---- round 1, local sums of exp relative to the chunk maxima ----
    {
      const float mpL = Mp * kLog2e, mqL = Mq * kLog2e;
      float sp = 0.0f, sq = 0.0f;
#pragma unroll
      for (int v = 0; v < NVMAX; ++v) {
        const int vi = vlo + v * kBlock + tid;
        if (vi < vhi) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            sp += __builtin_amdgcn_exp2f(__builtin_fmaf(T::at(xp[v], e), kLog2e, -mpL));
            sq += __builtin_amdgcn_exp2f(__builtin_fmaf(T::at(xq[v], e), kLog2e, -mqL));
          }
        }
      }
      sp = wsum(sp);
      sq = wsum(sq);
      if (lane == 0) {
        sm.f[wid][2] = sp;
        sm.f[wid][3] = sq;
      }
      __syncthreads();
      if (tid == 0) {
        const float Sp = (sm.f[0][2] + sm.f[1][2]) + (sm.f[2][2] + sm.f[3][2]);
        const float Sq = (sm.f[0][3] + sm.f[1][3]) + (sm.f[2][3] + sm.f[3][3]);
        tput(my_slot + 0, tag, __float_as_uint(Mp));
        tput(my_slot + 1, tag, (uint32_t)Ap);
        tput(my_slot + 2, tag, __float_as_uint(Sp));
        tput(my_slot + 3, tag, __float_as_uint(Mq));
        tput(my_slot + 4, tag, __float_as_uint(Sq));
      }
    }

    // ---- round 1, exchange: row lse_p, lse_q and argmax ----
    if (wid == 0) {
      uint64_t w[5] = {0, 0, 0, 0, 0};
      Waiter wt(a.ctl, a.timeout_ticks);
      for (;;) {
        bool ok = true;
        if (lane < a.C) {
#pragma unroll
          for (int j = 0; j < 5; ++j) {
            w[j] = tget(slot_row + lane * kSlotWords + j);
            ok = ok && tag_ok(w[j], tag);
          }
        }
        if (__all(ok)) break;
        if (!__all(wt.keep_going())) break;
      }
      float pm = -INFINITY, qm = -INFINITY, ps = 0.0f, qs = 0.0f;
      int pi = INT_MAX;
      if (lane < a.C) {
        pm = lo_f(w[0]);
        pi = (int)(uint32_t)w[1];
        ps = lo_f(w[2]);
        qm = lo_f(w[3]);
        qs = lo_f(w[4]);
      }
      float Mpr = pm;
      int A = pi;
      wargmax(Mpr, A);
      const float Mqr = wmax(qm);
      double tp = (lane < a.C) ? (double)ps * exp((double)pm - (double)Mpr) : 0.0;
      double tq = (lane < a.C) ? (double)qs * exp((double)qm - (double)Mqr) : 0.0;
      tp = wsumd(tp);
      tq = wsumd(tq);
      if (lane == 0) {
        const double lse_p = (double)Mpr + log(tp);
        const double lse_q = (double)Mqr + log(tq);
        sm.rf[0] = (float)lse_p;
        sm.rf[1] = (float)lse_q;
        sm.ri = A;
        sm.rd[0] = lse_q;
      }
    }
    __syncthreads();
    const float lse_p32 = sm.rf[0], lse_q32 = sm.rf[1];
    const int A = sm.ri;

    // ---- round 2, local: clipped reverse-KL terms and S ----
    const RowK rk = row_consts(lse_p32, lse_q32, a.tau);
    float qv[NVMAX][VEC], gv[NVMAX][VEC];
    float klc = 0.0f, ss = 0.0f;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      const int vi = vlo + v * kBlock + tid;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        qv[v][e] = 0.0f;
        gv[v][e] = 0.0f;
      }
      if (vi < vhi) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float q, r, g;
          opd_entry(T::at(xp[v], e), T::at(xq[v], e), rk, q, r, g);
          qv[v][e] = q;
          gv[v][e] = g;
          klc += __builtin_amdgcn_fmed3f(r, -a.tau, a.tau);
          ss += g;
        }
      }
    }
    klc = wsum(klc);
    ss = wsum(ss);
    if (lane == 0) {
      sm.f[wid][0] = klc;
      sm.f[wid][1] = ss;
    }
    __syncthreads();
    if (tid == 0) {
      const float kc = (sm.f[0][0] + sm.f[1][0]) + (sm.f[2][0] + sm.f[3][0]);
      const float sc = (sm.f[0][1] + sm.f[1][1]) + (sm.f[2][1] + sm.f[3][1]);
      tput(my_slot + 5, tag, __float_as_uint(kc));
      tput(my_slot + 6, tag, __float_as_uint(sc));
    }

    // ---- round 2, exchange: row KLc and S ----
    if (a.grad || owner) {
      if (wid == 0) {
        uint64_t w5 = 0, w6 = 0;
        Waiter wt(a.ctl, a.timeout_ticks);
        for (;;) {
          bool ok = true;
          if (lane < a.C) {
            w5 = tget(slot_row + lane * kSlotWords + 5);
            w6 = tget(slot_row + lane * kSlotWords + 6);
            ok = tag_ok(w5, tag) && tag_ok(w6, tag);
          }
          if (__all(ok)) break;
          if (!__all(wt.keep_going())) break;
        }
        double kk = (lane < a.C) ? (double)lo_f(w5) : 0.0;
        double s2 = (lane < a.C) ? (double)lo_f(w6) : 0.0;
        kk = wsumd(kk);
        s2 = wsumd(s2);
        if (lane == 0) {
          sm.rd[1] = kk;
          sm.rf[2] = (float)s2;
        }
      }
      __syncthreads();
    }

    // ---- gradient from the register-resident q and g ----
    if (a.grad) {
      const GradK gk = grad_consts(a.lam, a.gs, sm.rf[2]);
      const int va = A / VEC, ea = A - va * VEC;
      const int rel = va - vlo;
      const bool mine = va >= vlo && va < vhi && (rel & (kBlock - 1)) == tid;
      const int vown = rel / kBlock;
#pragma unroll
      for (int v = 0; v < NVMAX; ++v) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) qv[v][e] = grad_entry(qv[v][e], gv[v][e], gk);
      }
      if (mine) {
#pragma unroll
        for (int v = 0; v < NVMAX; ++v) {
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            if (v == vown && e == ea) qv[v][e] = qv[v][e] - gk.fix;
        }
      }
#pragma unroll
      for (int v = 0; v < NVMAX; ++v) {
        const int vi = vlo + v * kBlock + tid;
        if (vi < vhi) store_vec<VEC>(a.grad, (rowv + vi) * VEC, qv[v]);
      }
    }

    if (owner && tid == 0) {
      // A is in [0, V) unless a wait timed out on stale words; keep the read
      // inside the row either way.
      const int Ain = min(max(A, 0), a.V - 1);
      const float zqa = T::elem(a.zq, (long long)row * a.V + Ain);
      const double ce = sm.rd[0] - (double)zqa;
      const double kl = sm.rd[1];
      const double loss = (double)a.lam * ce + (1.0 - (double)a.lam) * kl;
      const float lf = (float)loss;
      a.row_loss[row] = lf;
      a.tgt[row] = A;
      if (a.stats)
        *(f32x4*)(a.stats + 4 * (long long)row) = (f32x4){lse_p32, lse_q32, sm.rf[2], (float)kl};
      tput(a.rowres + 2 * (long long)row, tag, (uint32_t)A);
      tput(a.rowres + 2 * (long long)row + 1, tag, __float_as_uint(lf));
    }
  }

  if (last_of_req) {
    __syncthreads();
    finish_request(a, s_off, req, tag);
  }
  if (item == a.n_items - 1u) {
    __syncthreads();
    finish_total(a, sm, tag);
  }
}

template <int VAR>
__global__ __launch_bounds__(kBlock) void fused_kernel(FwdArgs a) {
  extern __shared__ int s_off[];  // ragged row offsets [B + 1]
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const uint32_t epoch =
        (uint32_t)__hip_atomic_load(a.ctl + 1, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    sm.tag = epoch + 1u;  // epochs stay below 0xFFFFFFFF, so tags are never 0
  }
  int bad = 0;
  if (a.ragged) {
    for (int j = tid; j <= a.B; j += kBlock) s_off[j] = a.row_off[j];
    __syncthreads();
    int okl = 1;
    for (int j = tid; j < a.B; j += kBlock) {
      const int n = s_off[j + 1] - s_off[j];
      if (n < 1 || n > a.k) okl = 0;
    }
    if (tid == 0 && (s_off[0] != 0 || s_off[a.B] != a.R)) okl = 0;
    bad = !__syncthreads_and(okl);
    if (bad && tid == 0) raise_status(a.ctl, AV_DEV_BAD_OFFSETS);
  }
  __syncthreads();
  const uint32_t tag = sm.tag;
  for (;;) {
    if (tid == 0) {
      const uint64_t old =
          __hip_atomic_fetch_add(a.ctl, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.item = (uint32_t)old;
      sm.stat = (uint32_t)(old >> 32);
    }
    __syncthreads();
    const uint32_t item = sm.item, stat = sm.stat;
    __syncthreads();
    if (item >= a.n_items) {
      // The last take of the launch: every other workgroup has finished, so
      // the counter, the status and the epoch can be reset for the next one.
      if (tid == 0 && item == a.n_items + gridDim.x - 1u) {
        if (a.status_out) a.status_out[0] = (int32_t)(stat | (bad ? AV_DEV_BAD_OFFSETS : 0u));
        __hip_atomic_store(a.ctl, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t epoch = tag - 1u;
        const uint32_t next = (epoch + 1u == 0xFFFFFFFFu) ? 0u : epoch + 1u;
        __hip_atomic_store(a.ctl + 1, (uint64_t)next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    if (bad || stat != 0u) continue;  // failed launch: drain without work
    process_item<VAR>(a, sm, s_off, item, tag);
  }
}

// ---------------------------------------------------------------------------
// standalone backward
// ---------------------------------------------------------------------------

template <int VAR>
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
  const int vlo = (int)((long long)chunk * a.nvec / a.C);
  const int vhi = (int)((long long)(chunk + 1) * a.nvec / a.C);
  if (!verified) {
    float z[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) z[e] = 0.0f;
#pragma unroll
    for (int v = 0; v < NVMAX; ++v) {
      const int vi = vlo + v * kBlock + tid;
      if (vi < vhi) store_vec<VEC>(a.grad, (rowv + vi) * VEC, z);
    }
    return;
  }
  const f32x4 st = *(const f32x4*)(a.stats + 4 * (long long)row);
  const int A = a.tgt[row];
  const RowK rk = row_consts(st[0], st[1], a.tau);
  const GradK gk = grad_consts(a.lam, a.gs, st[2]);
  S xp[NVMAX], xq[NVMAX];
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
      xp[v] = T::load(a.zp, rowv + vi);
      xq[v] = T::load(a.zq, rowv + vi);
    }
  }
#pragma unroll
  for (int v = 0; v < NVMAX; ++v) {
    const int vi = vlo + v * kBlock + tid;
    if (vi < vhi) {
      float out[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float q, r, g;
        opd_entry(T::at(xp[v], e), T::at(xq[v], e), rk, q, r, g);
        out[e] = grad_entry(q, g, gk);
        if (vi * VEC + e == A) out[e] = out[e] - gk.fix;
      }
      store_vec<VEC>(a.grad, (rowv + vi) * VEC, out);
    }
  }
}

// ---------------------------------------------------------------------------
// length head and workspace fill
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void head_kernel(HeadArgs a) {
  __shared__ double s[kWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* hb = a.h + (long long)b * a.H;
  double acc = 0.0;
  for (int j = tid; j < a.H; j += kBlock) acc = fma((double)hb[j], (double)a.w[j], acc);
  acc = wsumd(acc);
  if ((tid & 63) == 0) s[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    const double z = ((s[0] + s[1]) + (s[2] + s[3])) + (double)a.bias;
    double sg;
    if (z >= 0.0) {
      sg = 1.0 / (1.0 + exp(-z));
    } else {
      const double e = exp(z);
      sg = e / (1.0 + e);
    }
    const double x = (double)a.gamma * sg * (double)a.k;
    const double n = a.mode == 0 ? ceil(x) : floor(x);
    const int bk = n < 1.0 ? 1 : (n > (double)a.k ? a.k : (int)n);
    a.bk[b] = bk;
    if (a.rate) a.rate[b] = (float)sg;
  }
}

__global__ __launch_bounds__(kBlock) void zero_kernel(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (size_t)gridDim.x * kBlock)
    p[i] = 0ull;
}

template <int VAR>
hipError_t launch_fused_t(const FwdArgs& a, int grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL(fused_kernel<VAR>, dim3(grid), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}
template <int VAR>
hipError_t occ_t(size_t lds, int* out) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, fused_kernel<VAR>, kBlock, lds);
}
template <int VAR>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.R * (unsigned)a.C;
  hipLaunchKernelGGL(bwd_kernel<VAR>, dim3(grid), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused(Variant v, const FwdArgs& a, int grid, size_t lds, hipStream_t s) {
  switch (v) {
    case kBf16x8: return launch_fused_t<kBf16x8>(a, grid, lds, s);
    case kBf16x1: return launch_fused_t<kBf16x1>(a, grid, lds, s);
    case kF32x4: return launch_fused_t<kF32x4>(a, grid, lds, s);
    default: return launch_fused_t<kF32x1>(a, grid, lds, s);
  }
}

hipError_t fused_blocks_per_cu(Variant v, size_t lds, int* out) {
  switch (v) {
    case kBf16x8: return occ_t<kBf16x8>(lds, out);
    case kBf16x1: return occ_t<kBf16x1>(lds, out);
    case kF32x4: return occ_t<kF32x4>(lds, out);
    default: return occ_t<kF32x1>(lds, out);
  }
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

hipError_t launch_zero(uint64_t* p, size_t words, hipStream_t s) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + kBlock - 1) / kBlock;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, words);
  return hipGetLastError();
}

}  // namespace avk
