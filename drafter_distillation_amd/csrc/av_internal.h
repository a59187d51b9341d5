// Internal interface between the C ABI (av_api.hip) and the gfx950 kernels
// (av_kernels.hip).  Not installed; callers use include/av.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avk {

constexpr int kBlock = 256;      // threads per workgroup of the streaming kernels
constexpr int kRowBlock = 1024;  // threads per workgroup of the fused row kernel (1 per CU)
constexpr int kMaxChunks = 64;   // chunks per row of the standalone backward

// Fused-pass workspace (64-bit words):
//   ctl[0]   status bits (high 32 bits) | row dispense counter (low 32 bits)
//   ctl[1]   launch epoch (low 32 bits)
//   ctl[2]   status bits (high 32 bits) | workgroups finished (low 32 bits)
//   rowres   [R][2]   per-row target argmax and loss (tagged)
//   reqres   [B][2]   per-request loss sum, float64 halves (tagged)
//   arrive   [B]      per-request count of completed verified rows (tagged)
//   halfres  [R][4][2] per part (half or quarter) of an unverified row: max
//                     of zp, its index (tagged)
//   harrive  [R]      per-row count of completed parts (tagged)
//   xres     [R][4][12] split rows: what each part (half or quarter) of a
//                     verified row hands the others (tagged): 8 words of
//                     first-sweep statistics, then 4 words of clip corrections
constexpr size_t kCtlBytes = 256;
constexpr int kXWords = 12;  // exchange words per part of a row
constexpr int kMaxParts = 4;  // parts of a split row

inline size_t ws_rowres_off() { return kCtlBytes; }
inline size_t ws_reqres_off(int R) { return ws_rowres_off() + (size_t)R * 16; }
inline size_t ws_arrive_off(int B, int R) { return ws_reqres_off(R) + (size_t)B * 16; }
inline size_t ws_halfres_off(int B, int R) { return ws_arrive_off(B, R) + (size_t)B * 8; }
inline size_t ws_harrive_off(int B, int R) { return ws_halfres_off(B, R) + (size_t)R * 64; }
inline size_t ws_xres_off(int B, int R) { return ws_harrive_off(B, R) + (size_t)R * 8; }
inline size_t ws_total(int B, int R) {
  size_t n = ws_xres_off(B, R) + (size_t)R * kMaxParts * kXWords * 8;
  return (n + 255) & ~(size_t)255;
}

// Longest-first row order of the dense layout needs B bytes of b_k and B
// 16-bit request indices in LDS; above this many requests rows go in index order.
constexpr int kMaxLptRequests = 4095;

// Kernel variants: element type and 16-byte vector width (or scalar access
// for rows that are not 16-byte aligned).
enum Variant { kBf16x8 = 0, kBf16x1 = 1, kF32x4 = 2, kF32x1 = 3 };

inline int variant_vec(Variant v) { return v == kBf16x8 ? 8 : v == kF32x4 ? 4 : 1; }
// Streaming backward: most vectors one thread holds per chunk.
inline int variant_nvmax(Variant v) { return v == kBf16x8 ? 8 : v == kF32x4 ? 8 : 16; }
// Fused row kernel: vectors per thread kept in registers and in LDS (16-byte
// vectors: 9 in registers use 72 of the 128 VGPRs a 1024-thread workgroup
// allows; 4 in LDS, for zp and zq, use 128 KB of the 160 KB).
#ifndef AV_NR
#define AV_NR 9
#endif
#ifndef AV_NL
#define AV_NL 4
#endif
constexpr int kRowRegs16 = AV_NR, kRowLds16 = AV_NL;
// Split rows (each verified row's halves on two CUs): register slots of a half
// whose 9..12 full slots fit on chip with 5 in registers and 4 in LDS (a
// 151936-wide bfloat16 row: 9.3 slots per half); halves of 13 slots and more
// use the whole-row split above.
constexpr int kPairRegs = 5;
// Smallest half-row (full 1024-vector slots) that the split form takes.
constexpr int kPairMinSlots = kPairRegs + AV_NL;
constexpr int kRowRegs1 = 32, kRowLds1 = 0;  // scalar variants
inline int variant_row_regs(Variant v) { return (v == kBf16x8 || v == kF32x4) ? kRowRegs16 : kRowRegs1; }
inline int variant_row_lds(Variant v) { return (v == kBf16x8 || v == kF32x4) ? kRowLds16 : kRowLds1; }

struct FwdArgs {
  const void* zp;
  const void* zq;
  const int32_t* draft;
  const int32_t* bk;
  const int32_t* row_off;
  int32_t* tgt;
  int32_t* acc;
  float* row_loss;
  float* req_loss;
  float* total;
  float* stats;
  void* grad;     // [R, V] float32, or bfloat16 when gbf16
  int32_t* status_out;
  uint64_t* ctl;
  uint64_t* rowres;
  uint64_t* reqres;
  uint64_t* arrive;
  uint64_t* halfres;
  uint64_t* harrive;
  uint64_t* xres;
  long long timeout_ticks;
  int B, k, V, R;
  int nvec;      // vectors per row (V / vec)
  int nr, nl;    // vectors per thread held in registers / in LDS
  int ragged;
  int lpt;       // dense layout, rows handed out longest first (unverified rows in halves)
  int split;     // 1: whole rows; 2: rows in halves on workgroup pairs (2p, 2p+1), each
                 // half kept on chip; 3: rows 0 .. nwhole-1 whole, the rest in halves
                 // (ragged layout), all claimed from the dispenser; 4: rows in
                 // quarters on teams of four workgroups (4t .. 4t+3)
  int pv0;       // split 2 and 3: first vector of the second half
  int nwhole;    // split 3: rows taken whole
  int nquart;    // longest-first dense layout, split 1: at most this many of the
                 // last unverified rows are handed out in quarters (the rest in halves)
  int gbf16;     // gradient stored as bfloat16
  float lam, tau, gs;
  // temperature of the reverse-KL term
  float* lse1;          // [R] log-sum-exp of zq at temperature 1, or NULL
  int tm;               // T differs from 1
  float inv_t, inv_tl;  // 1 / T and log2(e) / T (float32 roundings of the float64 values)
};

struct BwdArgs {
  const void* zp;
  const void* zq;
  const int32_t* bk;
  const int32_t* tgt;
  const float* stats;
  const float* lse1;  // [R] log-sum-exp of zq at temperature 1 (read when tm)
  void* grad;  // float32, or bfloat16 when gbf16
  int B, k, V, R, C, nvec, ragged, gbf16, tm;
  float lam, tau, gs;
  float inv_t, inv_tl;
};

struct HeadArgs {
  const float* h;
  const float* w;
  float* rate;
  int32_t* bk;
  float bias, gamma;
  int B, H, k, mode;
};

struct HeadUpdArgs {
  const float* h;
  const int32_t* acc;
  const int32_t* bk;
  float* w;
  float* bias;
  float* m_w;
  float* v_w;
  float* m_b;
  float* v_b;
  float* loss;
  float* rate;
  float* grad_h;
  double* ws;  // [2B]: d loss / d z_b, then the squared errors
  int B, H, k;
  double lr, beta1, beta2, eps, wd;
  double bc1, sqrt_bc2;  // 1 - beta1^t, sqrt(1 - beta2^t)
};

struct SpecArgs {
  const void* zp;
  const void* zq;
  const int32_t* draft;
  const int32_t* bk;
  const int32_t* row_off;
  const float* u;
  int32_t* acc;
  int32_t* token;
  float* stats;     // [R, 2] lse_p, lse_q of verified rows, or NULL
  const float* stats_in;  // [R, stats_stride] lse_p, lse_q given by the caller, or NULL
  int stats_stride;
  int32_t* status;  // [1] or NULL
  uint32_t* ws;     // [R][4]: accepted flag, lse_p bits, lse_q bits
  uint32_t* chunks; // [B][nchunk][4]: best residual key and index, best p key and index
  uint64_t seed;
  int B, k, V, R, nvec, ragged;
  int chunk, nchunk;  // vectors per chunk of the race, chunks per row (<= kSpecMaxChunks)
};
constexpr int kSpecMaxChunks = 64;
// Fewest vectors per chunk of the race (512: 38 chunks of a 151936-wide bf16
// row, enough workgroups to keep the generator's arithmetic busy; 2048 was
// 3% slower, 256 slower again).
constexpr int kSpecChunkVecs = 512;

// full: every on-chip slot of a row is filled (nvec >= (regs + lds) * kRowBlock)
// and the default on-chip split is used.
// a.tm selects the tempered form of the kernels (fused and backward).
// nr: register slots of the build (kRowRegs16, or kPairRegs for split rows).
// a.split (1, 2, 3 or 4) selects whole rows, rows in halves, whole rows with
// a split tail, or rows in quarters.
hipError_t launch_fused(Variant v, bool full, int nr, const FwdArgs& a, int grid, size_t lds, hipStream_t s);
hipError_t fused_blocks_per_cu(Variant v, bool full, int split, int nr, bool gbf16, bool tm, size_t lds, int* out);
hipError_t launch_bwd(Variant v, const BwdArgs& a, hipStream_t s);
hipError_t launch_head(const HeadArgs& a, hipStream_t s);
hipError_t launch_head_update(const HeadUpdArgs& a, hipStream_t s);
hipError_t launch_spec(Variant v, const SpecArgs& a, hipStream_t s);
hipError_t launch_zero(uint64_t* p, size_t words, hipStream_t s);

}  // namespace avk
