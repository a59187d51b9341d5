// Backward of the drafter's LM head (the step after the verify + OPD pass):
//   d_hid[r, h] = sum_v dz[r, v] W[v, h]        d_W[v, h] = sum_r dz[r, v] hid[r, h]
// Two bfloat16 GEMMs with float32 accumulation and output on the matrix
// cores of gfx950 (v_mfma_f32_32x32x16_bf16).  Semantics are documented in
// include/av.h.
//
// Both compute C[M, N] = A[M, K] B[K, N], C row-major float32.  A is
// K-contiguous (element (m, k) at A[m lda + k]) or M-contiguous (at
// A[k lda + m]); B is K-contiguous (B[n ldb + k]) or N-contiguous
// (B[k ldb + n]).  d_hid: A = dz (K-contiguous), B = W (N-contiguous);
// d_W: A = dz read as dz^T (M-contiguous), B = hid (N-contiguous).
// A workgroup of 256 threads (4 waves, 2 x 2) owns a 256 x 256 tile of C;
// each wave a 128 x 128 quarter: 4 x 4 blocks of 32 x 32, 256 float32
// accumulators per lane.  K advances 64 at a time through two LDS buffers.
//
// Operands are staged through registers: global loads run two K-steps ahead
// and are written to the free LDS buffer between the current step's products.
// A K-contiguous operand is held in LDS as [row][k] (rows padded to 72 values
// so that the lanes of a 16-byte fragment read fall on distinct banks); an M-
// or N-contiguous one as [k][row], as it lies in memory, with an XOR swizzle of
// its 16-byte chunks, and its fragments are read with the transposing LDS read
// ds_read_b64_tr_b16 (see frag_t).  Shapes without 16-byte rows load element
// by element and transpose 8 x 8 blocks in registers with byte permutes.
// Long K (d_hid: K = V) is split over workgroups; the partial tiles go to
// the workspace and reduce_kernel adds them in split order.  Tiles map to
// workgroup ids so that the 32 workgroups that run together on one XCD (ids
// equal mod 8) form an 8 x 4 block of tiles, which share operand slices in
// that XCD's L2 (see tile_of).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "av.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kLdk = kBK + 8;  // LDS row length (bfloat16 values)
constexpr int kThreads = 256;
constexpr int kMaxSplits = 8;
constexpr int kMaxDim = 1 << 30;  // largest R (tile offsets stay in int)
constexpr int kMaxLd = 1 << 22;   // largest V, H (per-thread buffer offsets stay in 31 bits)

thread_local char g_err[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_err, sizeof(g_err), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return AV_EHIP;
}

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  float* C;       // [M, N], or the splits' partial tiles [splits][M][N] when splits > 1
  long long lda, ldb;
  long long a_total, b_total;  // elements of A and B
  int M, N, K;
  int tiles_m, tiles_n, splits, kchunk;  // kchunk: K values per split (a multiple of kBK)
  int group;      // N tiles per group of the tile order (see tile_of)
  int per_xcd;    // tiles per XCD: ceil(tiles_m tiles_n splits / 8)
  int vec;        // rows 16-byte aligned and M, N, K multiples of 8 (kFast / kEdge loads)
};

// Workgroup id -> (tile_m, tile_n, split); false for ids past the last tile.
// Tiles are ordered split-major, then in groups of `group` N tiles, each group
// covering every M tile with its N tiles adjacent; XCD x (the workgroups with
// id % 8 == x) takes the x-th contiguous run of per_xcd tiles in that order,
// so the workgroups running together on one XCD share operand slices in its L2.
__device__ __forceinline__ bool tile_of(const GemmArgs& g, int id, int& tm, int& tn, int& sp) {
  const int v = (id & 7) * g.per_xcd + (id >> 3);
  const int tt = g.tiles_m * g.tiles_n;
  sp = v / tt;
  if (sp >= g.splits) return false;
  const int rem = v - sp * tt;
  const int grp = rem / (g.tiles_m * g.group);
  const int w = rem - grp * g.tiles_m * g.group;
  const int gs = min(g.group, g.tiles_n - grp * g.group);
  tn = grp * g.group + w % gs;
  tm = w / gs;
  return true;
}

// Load modes: kFast, a tile inside M, N and K on 16-byte aligned rows (no
// checks); kEdge, aligned rows with M, N and K multiples of 8, so that each
// 16-byte piece lies wholly inside or wholly outside (outside: zeros);
// kScalar, element by element, zeros outside.
enum Mode { kFast = 0, kEdge = 1, kScalar = 2 };

// 16-byte staging of one K-step: eight 16-byte pieces per thread per operand.
struct Stage {
  u32x4 v[8];
};

// Operands are read through buffer resources based at the K-step's corner of
// the tile: a thread's pieces then differ by wave-uniform offsets, and no
// 64-bit address is kept per piece.  The resource's extent is what is left
// of the operand, so no load reaches past its end.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc_at(const uint16_t* P, long long total, long long off) {
  const long long bytes = (total - off) * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(P + off), (short)0,
                                           bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint32_t ld16(Rsrc r, uint32_t vo, uint32_t so) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
}

// Where an operand lies: element (row, k) at P[row ld + k] (K-contiguous) or
// P[k ld + row] (row-contiguous); `total` elements; `rows` rows (M or N).
struct Opnd {
  const uint16_t* P;
  long long ld, total;
  int rows;
};

// K-contiguous operand, rows r0 .. r0+255, k0 .. k0+63: piece q of thread t is
// row t / 8 + 32 q, values 8 (t % 8) .. + 7 (eight threads cover one 128-byte
// row segment).
template <int MODE>
__device__ __forceinline__ void load_k(const Opnd& o, int r0, int k0, int kend, Stage& st) {
  const int tid = threadIdx.x, rr = tid >> 3, c = (tid & 7) * 8;
  const Rsrc r = rsrc_at(o.P, o.total, (long long)r0 * o.ld + k0);
  const uint32_t vo = (uint32_t)((rr * o.ld + c) * 2), step = (uint32_t)(32 * o.ld * 2);
  const int gk = k0 + c;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int gr = r0 + rr + 32 * q;
    if (MODE == kFast || (MODE == kEdge && gr < o.rows && gk < kend)) {
      st.v[q] = __builtin_amdgcn_raw_buffer_load_b128(r, vo, q * step, 0);
    } else if (MODE == kEdge) {
      st.v[q] = u32x4{0u, 0u, 0u, 0u};
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (gr < o.rows)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gk + e < kend) w[e >> 1] |= ld16(r, vo + 2 * e + q * step, 0) << (16 * (e & 1));
      st.v[q] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}
__device__ __forceinline__ void store_k1(const Stage& st, uint16_t* lds, int q) {
  const int tid = threadIdx.x;
  *(u32x4*)(lds + ((tid >> 3) + 32 * q) * kLdk + (tid & 7) * 8) = st.v[q];
}
__device__ __forceinline__ void store_k(const Stage& st, uint16_t* lds) {
#pragma unroll
  for (int q = 0; q < 8; ++q) store_k1(st, lds, q);
}

// Row-contiguous operand, rows r0 .. r0+255, k0 .. k0+63: thread t loads the
// 8 x 8 block of rows 8 (t / 8) .. + 7 and k values 8 (t % 8) .. + 7 as eight
// 16-byte pieces along the rows, one per k.
template <int MODE>
__device__ __forceinline__ void load_r(const Opnd& o, int r0, int k0, int kend, Stage& st) {
  const int tid = threadIdx.x, cb = (tid >> 3) * 8, kk = (tid & 7) * 8;
  const Rsrc r = rsrc_at(o.P, o.total, (long long)k0 * o.ld + r0);
  const uint32_t vo = (uint32_t)((kk * o.ld + cb) * 2), step = (uint32_t)(o.ld * 2);
  const int gr = r0 + cb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int gk = k0 + kk + i;
    if (MODE == kFast || (MODE == kEdge && gk < kend && gr < o.rows)) {
      st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, vo, i * step, 0);
    } else if (MODE == kEdge) {
      st.v[i] = u32x4{0u, 0u, 0u, 0u};
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (gk < kend)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gr + e < o.rows) w[e >> 1] |= ld16(r, vo + 2 * e + i * step, 0) << (16 * (e & 1));
      st.v[i] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}
// Transposes the thread's block (piece i = the 8 rows' values at k = i) into
// 8 rows of 8 k values and writes them to LDS rows 8 (t / 8) + c, columns
// 8 (t % 8) .. + 7.  Output word i of row c pairs k = 2i and 2i + 1: the low
// (c even) or high (c odd) halves of word c / 2 of pieces 2i and 2i + 1.
__device__ __forceinline__ void store_r(const Stage& st, uint16_t* lds) {
  const int tid = threadIdx.x;
  uint16_t* base = lds + ((tid >> 3) * 8) * kLdk + (tid & 7) * 8;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_perm(st.v[2 * i + 1][c >> 1], st.v[2 * i][c >> 1], sel);
    *(u32x4*)(base + c * kLdk) = o;
  }
}

// Row-contiguous operand kept as it lies, [k][row] in LDS (read back with
// transposing fragment reads, frag_t): thread t loads row chunk t % 32 (8
// rows, 16 bytes) of k-rows 8 (t / 32) .. + 7, so 32 lanes read one k-row's
// 512 bytes and the 8 lanes of each 128-byte LDS write share a k-row.
// k-row k's chunk c sits at position c ^ 4 (k % 4): the four k-rows that one
// transposing read serves then start on different banks.
template <int MODE>
__device__ __forceinline__ void load_rt(const Opnd& o, int r0, int k0, int kend, Stage& st) {
  static_assert(MODE != kScalar, "16-byte rows only");
  const int tid = threadIdx.x, c = tid & 31, kb = (tid >> 5) * 8;
  const Rsrc r = rsrc_at(o.P, o.total, (long long)k0 * o.ld + r0);
  const uint32_t vo = (uint32_t)((kb * o.ld + 8 * c) * 2), step = (uint32_t)(o.ld * 2);
  const bool cin = MODE == kFast || r0 + 8 * c < o.rows;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (MODE == kFast || (cin && k0 + kb + i < kend))
      st.v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, vo, i * step, 0);
    else
      st.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void store_rt1(const Stage& st, uint16_t* lds, int i) {
  const int tid = threadIdx.x, c = tid & 31, k = (tid >> 5) * 8 + i;
  *(u32x4*)(lds + k * 256 + 8 * (c ^ (4 * (k & 3)))) = st.v[i];
}
__device__ __forceinline__ void store_rt(const Stage& st, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < 8; ++i) store_rt1(st, lds, i);
}

// Matrix-core fragment of rows rb .. rb + 31, 16-wide k step s (lane l: row
// rb + l % 32, k values 8 (l / 32) .. + 7) from a [k][256] LDS block laid out
// by store_rt.  ds_read_b64_tr_b16 hands lane i of each 16-lane group value
// i % 4 of the 8-byte reads of lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4 (a probe established this), so four lanes reading 4 consecutive
// rows at 4 consecutive k give each lane 4 consecutive k of its own row; two
// such reads make the lane's 8 values.
__device__ __forceinline__ bf16x8 frag_t(const uint16_t* lds, int rb, int s) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int l = threadIdx.x & 63, g = l >> 4, i = l & 15;
  const int n = rb + 16 * (g & 1) + 4 * (i & 3);
  s16x4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 16 * s + 8 * (g >> 1) + 4 * h + (i >> 2);
    const uint16_t* p = lds + k * 256 + 8 * ((n >> 3) ^ (4 * (k & 3))) + (n & 7);
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  }
  // k values 0..3 of the lane's 8, then 4..7
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Scheduling of one 16-wide k step's 16 products: product q is followed by an
// LDS read if q < NR (the next k step's fragments, read early) and by an LDS
// write if q >= 16 - NW (the next K-step's operands, written late, so their
// global loads have had the most time).
template <int NR, int NW, int Q = 0>
__device__ __forceinline__ void sched_products() {
  if constexpr (Q < 16) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (Q < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if constexpr (Q >= 16 - NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    sched_products<NR, NW, Q + 1>();
  }
}

// One K-step's products from LDS buffer `buf`: each wave's 128 x 128 quarter,
// four 16-wide k steps of 4 x 4 matrix-core products.  AT, BT: A or B is
// held as [k][row] (store_rt) and read with transposing reads.  IL: the next
// K-step's operands (sa, sb: 8 pieces each, neither transposed in registers)
// are written to LDS buffers `nxt` between the products, two pieces of each
// per 16-wide k step.
template <bool AT, bool BT, int IL = 0>
__device__ __forceinline__ void products(const uint16_t (*buf)[kBM * kLdk], f32x16 (&acc)[4][4],
                                         const Stage* sa = nullptr, const Stage* sb = nullptr,
                                         uint16_t (*nxt)[kBM * kLdk] = nullptr) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // lane l reads row l % 32 of a 32-row block, k values 8 (l / 32) .. + 7 of a
  // 16-wide k step
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  const int bn = (wid & 1) * 128;
  const int am = (wid >> 1) * 128;
  const uint16_t* As = buf[0] + (am + frow) * kLdk + fk;
  const uint16_t* Bs = buf[1] + (bn + frow) * kLdk + fk;
  auto afrag = [&](int i, int s) {
    if constexpr (AT) return frag_t(buf[0], am + 32 * i, s);
    else return *(const bf16x8*)(As + i * 32 * kLdk + 16 * s);
  };
  auto bfrag = [&](int i, int s) {
    if constexpr (BT) return frag_t(buf[1], bn + 32 * i, s);
    else return *(const bf16x8*)(Bs + i * 32 * kLdk + 16 * s);
  };
  constexpr int kReads = (AT ? 8 : 4) + (BT ? 8 : 4);  // LDS reads of one 16-wide k step
  // IL 1: two pieces of each operand after each 16-wide k step's products;
  // IL 2: all sixteen after the last k step's (which reads nothing)
  constexpr int kWrites = IL == 1 ? 4 : 0;
  static_assert(kReads <= 16, "one read per product at most");
  // fragments of 16-wide k step s + 1 are read while step s's products run
  bf16x8 a[2][4], b[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[0][i] = afrag(i, 0);
    b[0][i] = bfrag(i, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
  for (int s = 0; s < kBK / 16; ++s) {
    const int c = s & 1;
    if (s + 1 < kBK / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[c ^ 1][i] = afrag(i, s + 1);
        b[c ^ 1][i] = bfrag(i, s + 1);
      }
    }
    if (IL == 1 || (IL == 2 && s + 1 == kBK / 16)) {
#pragma unroll
      for (int q = IL == 1 ? 2 * s : 0; q < (IL == 1 ? 2 * s + 2 : 8); ++q) {
        if constexpr (AT) store_rt1(*sa, nxt[0], q);
        else store_k1(*sa, nxt[0], q);
        if constexpr (BT) store_rt1(*sb, nxt[1], q);
        else store_k1(*sb, nxt[1], q);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
    if (s + 1 < kBK / 16) sched_products<kReads, kWrites>();
    else sched_products<0, IL == 2 ? 16 : kWrites>();
  }
}

template <bool AK, bool BK, int MODE, bool AT = false, bool BT = false>
struct Loader {
  const Opnd& a;
  const Opnd& b;
  int m0, n0, kbeg, kend;
  __device__ __forceinline__ void load(int t, Stage& sa, Stage& sb) const {
    const int k0 = kbeg + t * kBK;
    if constexpr (AK) load_k<MODE>(a, m0, k0, kend, sa);
    else if constexpr (AT) load_rt<MODE>(a, m0, k0, kend, sa);
    else load_r<MODE>(a, m0, k0, kend, sa);
    if constexpr (BK) load_k<MODE>(b, n0, k0, kend, sb);
    else if constexpr (BT) load_rt<MODE>(b, n0, k0, kend, sb);
    else load_r<MODE>(b, n0, k0, kend, sb);
  }
  __device__ __forceinline__ static void store(uint16_t (*buf)[kBM * kLdk], const Stage& sa, const Stage& sb) {
    if constexpr (AK) store_k(sa, buf[0]);
    else if constexpr (AT) store_rt(sa, buf[0]);
    else store_r(sa, buf[0]);
    if constexpr (BK) store_k(sb, buf[1]);
    else if constexpr (BT) store_rt(sb, buf[1]);
    else store_r(sb, buf[1]);
  }
};

// The K loop of one tile: acc += A[m0 .., kbeg .. kend) B[kbeg .. kend), n0 ..],
// through the two LDS buffers.  Global loads run two K-steps ahead of the
// products: step t + 2 is requested while step t's products run, and step
// t + 1 (requested one step earlier) is written to LDS between them.
template <bool AK, bool BK, int MODE, bool AT, bool BT>
__device__ __forceinline__ void k_loop2(const Loader<AK, BK, MODE, AT, BT>& L, uint16_t (*lds)[2][kBM * kLdk],
                                        f32x16 (&acc)[4][4]) {
  const int nk = (L.kend - L.kbeg + kBK - 1) / kBK;
  if (nk <= 0) return;
  // Branch-free trips: past the last step, loads repeat the last step (in
  // bounds, unused) and stores go to a buffer that is not read again.
  const int last = nk - 1;
  Stage s0a, s0b, s1a, s1b;
  L.load(0, s0a, s0b);
  L.store(lds[0], s0a, s0b);
  L.load(min(1, last), s1a, s1b);
  __syncthreads();
  // two steps per trip, so that each register stage is a fixed set of registers;
  // at the top of a trip LDS buffer 0 holds step t and stage 1 step t + 1
  // Where the next step's LDS writes go among the products (measured at
  // R=2048, V=151936, H=4096): with one K-contiguous operand (d_hid, 12
  // fragment reads per 16-wide k step) spread over the k steps, 1255 against
  // 1180 TFLOP/s when written after the products; with none (d_W, 16 reads)
  // after the last k step's products, which read nothing.
  constexpr int IL = AK || BK ? 1 : 2;
  int t = 0;
  for (; t + 1 < nk; t += 2) {
    L.load(min(t + 2, last), s0a, s0b);
    products<AT, BT, IL>(lds[0], acc, &s1a, &s1b, lds[1]);
    __syncthreads();
    L.load(min(t + 3, last), s1a, s1b);
    products<AT, BT, IL>(lds[1], acc, &s0a, &s0b, lds[0]);
    __syncthreads();
  }
  if (t < nk) products<AT, BT>(lds[0], acc);  // odd step count: the last step
}

// The same with loads one K-step ahead (element-wise loads: fewer registers).
template <bool AK, bool BK, int MODE, bool AT, bool BT>
__device__ __forceinline__ void k_loop1(const Loader<AK, BK, MODE, AT, BT>& L, uint16_t (*lds)[2][kBM * kLdk],
                                        f32x16 (&acc)[4][4]) {
  const int nk = (L.kend - L.kbeg + kBK - 1) / kBK;
  if (nk <= 0) return;
  Stage sa, sb;
  L.load(0, sa, sb);
  L.store(lds[0], sa, sb);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) L.load(t + 1, sa, sb);
    products<AT, BT>(lds[t & 1], acc);
    if (t + 1 < nk) L.store(lds[(t + 1) & 1], sa, sb);
    __syncthreads();
  }
}

// Writes a workgroup's accumulators: register r of block (i, j) of wave
// (wm, wn) is row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32 of that
// block.  Partial tiles of a split sum go to the split's slice of the workspace.
__device__ __forceinline__ void store_tile(const GemmArgs& g, const f32x16 (&acc)[4][4], int m0, int n0, int sp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  float* C = g.C + (g.splits > 1 ? (long long)sp * g.M * g.N : 0);
  const int col0 = n0 + wn * 128 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row < g.M) {
        float* crow = C + (long long)row * g.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = col0 + j * 32;
          if (col < g.N) __builtin_nontemporal_store(acc[i][j][r], crow + col);
        }
      }
    }
}

template <bool AK, bool BK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kBM * kLdk];  // [buffer][A, B]
  int tm, tn, sp;
  if (!tile_of(g, blockIdx.x, tm, tn, sp)) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int kbeg = sp * g.kchunk, kend = min(g.K, kbeg + g.kchunk);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  const Opnd oa{g.A, g.lda, g.a_total, g.M}, ob{g.B, g.ldb, g.b_total, g.N};
  // 16-byte rows: an operand that is not K-contiguous stays as it lies in
  // LDS and is read with transposing reads (no register transposes)
  constexpr bool AT = !AK, BT = !BK;
  if (!g.vec) {
    k_loop1(Loader<AK, BK, kScalar>{oa, ob, m0, n0, kbeg, kend}, lds, acc);
  } else if (m0 + kBM <= g.M && n0 + kBN <= g.N) {
    // whole K-steps unchecked, then the partial last one (if any) checked
    const int kfull = kend > kbeg ? kbeg + (kend - kbeg) / kBK * kBK : kbeg;
    k_loop2(Loader<AK, BK, kFast, AT, BT>{oa, ob, m0, n0, kbeg, kfull}, lds, acc);
    if (kfull < kend) k_loop1(Loader<AK, BK, kEdge, AT, BT>{oa, ob, m0, n0, kfull, kend}, lds, acc);
  } else {
    k_loop2(Loader<AK, BK, kEdge, AT, BT>{oa, ob, m0, n0, kbeg, kend}, lds, acc);
  }

  store_tile(g, acc, m0, n0, sp);
}

// C = sum over splits of the partial tiles, in split order.
__global__ __launch_bounds__(256) void reduce_kernel(const float* part, float* C, long long n, int splits) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    float s = part[i];
    for (int q = 1; q < splits; ++q) s += part[(long long)q * n + i];
    C[i] = s;
  }
}

template <bool AK, bool BK>
hipError_t launch_gemm(GemmArgs& g, bool vec, hipStream_t s) {
  const long long tiles = (long long)g.tiles_m * g.tiles_n * g.splits;
  if (tiles > 0x7ffffff0LL) return hipErrorInvalidValue;
  g.per_xcd = (int)((tiles + 7) / 8);
  const dim3 grid((unsigned)(8LL * g.per_xcd));
  g.vec = vec;
  hipLaunchKernelGGL((gemm_kernel<AK, BK>), grid, dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Splits of d_hid's long K: enough workgroups for the device (about one per
// CU), a K range per split that is a multiple of kBK.
int hid_splits(int R, int V, int H, int cus) {
  const long long tiles = ((long long)R + kBM - 1) / kBM * (((long long)H + kBN - 1) / kBN);
  int s = 1;
  while (s < kMaxSplits && tiles * s * 2 <= cus && (long long)V / (2 * s) >= 8 * kBK) s *= 2;
  if (tiles * s < cus && s < kMaxSplits && (long long)V / (2 * s) >= 8 * kBK) s *= 2;
  return s;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) return 256;
  return cus;
}

}  // namespace

extern "C" {

size_t av_lm_head_workspace_bytes(int R, int V, int H) {
  if (R < 1 || V < 1 || H < 1 || R > kMaxDim || V > kMaxLd || H > kMaxLd) return 0;
  const int s = hid_splits(R, V, H, device_cus());
  return s > 1 ? (size_t)s * R * H * sizeof(float) : 0;
}

int av_lm_head_bwd(int R, int V, int H, const void* dz, const void* w, const void* hid, float* d_hid,
                   float* d_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (R < 1 || V < 1 || H < 1 || !dz) return AV_EINVAL;
  if (R > kMaxDim || V > kMaxLd || H > kMaxLd) return AV_EUNSUPPORTED;
  if ((d_hid && !w) || (d_w && !hid)) return AV_EINVAL;
  if (workspace_bytes > 0 && !workspace) return AV_EINVAL;
  const hipStream_t s = (hipStream_t)stream;
  // 16-byte loads need every row start, and every edge of M, N and K, on an
  // 8-value bound
  const bool vec = R % 8 == 0 && V % 8 == 0 && H % 8 == 0 && aligned16(dz) && (!w || aligned16(w)) &&
                   (!hid || aligned16(hid));
  if (d_hid) {
    GemmArgs g{};
    g.A = (const uint16_t*)dz;
    g.lda = V;
    g.a_total = (long long)R * V;
    g.B = (const uint16_t*)w;
    g.ldb = H;
    g.b_total = (long long)V * H;
    g.M = R;
    g.N = H;
    g.K = V;
    g.tiles_m = (R + kBM - 1) / kBM;
    g.tiles_n = (H + kBN - 1) / kBN;
    int splits = hid_splits(R, V, H, device_cus());
    if ((size_t)splits * R * H * sizeof(float) > workspace_bytes || !aligned16(workspace)) splits = 1;
    g.splits = splits;
    g.kchunk = (int)((((long long)V + splits - 1) / splits + kBK - 1) / kBK * kBK);
    g.group = g.tiles_n < 4 ? g.tiles_n : 4;
    g.C = splits > 1 ? (float*)workspace : d_hid;
    hipError_t e = launch_gemm<true, false>(g, vec, s);
    if (e == hipSuccess && splits > 1) {
      const long long n = (long long)R * H;
      const long long blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
      hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)workspace, d_hid,
                         n, splits);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return hip_fail(e);
  }
  if (d_w) {
    GemmArgs g{};
    g.A = (const uint16_t*)dz;  // dz^T: element (v, r) at dz[r V + v]
    g.lda = V;
    g.a_total = (long long)R * V;
    g.B = (const uint16_t*)hid;
    g.ldb = H;
    g.b_total = (long long)R * H;
    g.M = V;
    g.N = H;
    g.K = R;
    g.tiles_m = (V + kBM - 1) / kBM;
    g.tiles_n = (H + kBN - 1) / kBN;
    g.splits = 1;
    g.kchunk = (R + kBK - 1) / kBK * kBK;
    g.group = g.tiles_n < 4 ? g.tiles_n : 4;
    g.C = d_w;
    const hipError_t e = launch_gemm<false, false>(g, vec, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return AV_OK;
}

const char* av_lm_head_last_error(void) { return g_err; }

}  // extern "C"
