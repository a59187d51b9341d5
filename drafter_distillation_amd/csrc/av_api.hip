// C ABI of the verify + OPD library: host-side argument checks, launch
// configuration, error reporting.  Semantics are documented in include/av.h.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "av.h"
#include "av_internal.h"
#include "av_test.h"

namespace {

thread_local char g_hip_err[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_err, sizeof(g_hip_err), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return AV_EHIP;
}

// Per-device launch facts, queried once per device and variant.
struct DeviceInfo {
  int cus = 0;
  long long ticks_per_ms = 0;  // wall-clock counter rate
  int occ[4][8][2][2] = {};    // fused-kernel workgroups per CU, per variant, kernel form
                               // (see kForms), gradient type and plain/tempered form, with
                               // the most dynamic LDS a launch uses
};
// Kernel forms: {fast form, split (1 whole rows, 2 split rows, 3 split
// tail, 4 rows in quarters), register slots of the build}.
struct FormDesc {
  bool full;
  int split, nr;
};
constexpr int kNumForms = 8;
constexpr FormDesc kForms[kNumForms] = {{false, 1, 0}, {true, 1, 0}, {false, 2, avk::kRowRegs16},
                                        {true, 2, avk::kRowRegs16}, {true, 2, avk::kPairRegs},
                                        {false, 3, avk::kRowRegs16}, {true, 3, avk::kRowRegs16},
                                        {false, 4, avk::kRowRegs16}};
int form_index(bool full, int split, int nr) {
  if (split == 4) return 7;
  if (split == 3) return full ? 6 : 5;
  if (split != 2) return full ? 1 : 0;
  if (!full) return 2;
  return nr == avk::kPairRegs ? 4 : 3;
}
// Most dynamic LDS of a fused launch: ragged offsets of 4095 requests, or the
// longest-first schedule of avk::kMaxLptRequests requests.
constexpr size_t kMaxDynLds = 4096 * sizeof(int32_t);
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];
hipError_t g_dev_err[kMaxDevices];

hipError_t device_info(const DeviceInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_dev_once[dev], [dev]() {
    DeviceInfo& d = g_dev[dev];
    hipError_t err = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    int khz = 0;
    if (err == hipSuccess) err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    d.ticks_per_ms = khz > 0 ? (long long)khz : 100000;
    for (int v = 0; v < 4 && err == hipSuccess; ++v)
      for (int f = 0; f < kNumForms && err == hipSuccess; ++f)
        for (int g = 0; g < 2 && err == hipSuccess; ++g)
          for (int t = 0; t < 2 && err == hipSuccess; ++t)
            err = avk::fused_blocks_per_cu((avk::Variant)v, kForms[f].full, kForms[f].split, kForms[f].nr,
                                           g != 0, t != 0, kMaxDynLds, &d.occ[v][f][g][t]);
    g_dev_err[dev] = err;
  });
  if (g_dev_err[dev] != hipSuccess) return g_dev_err[dev];
  *out = &g_dev[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace of av_verify_opd_fwd_noalloc: one array per GPU, resident from
// the library's load to the end of the process.  Its host-side name is only a
// handle: kernels get the device address that hipGetSymbolAddress returns for
// the current device, looked up (and the array zeroed) once per device.
static __device__ __align__(256) unsigned char scratch[AV_NOALLOC_SCRATCH_BYTES];
void* g_scratch[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    // zeroed once, synchronously: the pass's launch epoch and tagged words
    // start from zero; every later call leaves the array ready for the next
    if (err == hipSuccess) err = hipMemset(p, 0, AV_NOALLOC_SCRATCH_BYTES);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    g_scratch[dev] = err == hipSuccess ? p : nullptr;
    g_scratch_err[dev] = err;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch[dev];
  return hipSuccess;
}

// Shared validation of the verify entry points.  Fills the layout facts.
struct Plan {
  avk::Variant var;
  int vec, nvec;
  bool ragged;
};

int plan_rows(int dtype, int B, int k, int V, int R, const int32_t* row_off, const void* zp,
              const void* zq, const void* grad, Plan* p) {
  if (dtype != AV_F32 && dtype != AV_BF16) return AV_EUNSUPPORTED;
  if (B < 1 || k < 1 || k > AV_MAX_K || V < 1 || R < 1) return AV_EINVAL;
  p->ragged = row_off != nullptr;
  if (!p->ragged && (long long)R != (long long)B * k) return AV_EINVAL;
  if (p->ragged && ((long long)R < B || (long long)R > (long long)B * k)) return AV_EINVAL;
  const int vec = dtype == AV_BF16 ? 8 : 4;
  const bool vec_ok = V % vec == 0 && aligned16(zp) && aligned16(zq) && (grad == nullptr || aligned16(grad));
  if (dtype == AV_BF16) p->var = vec_ok ? avk::kBf16x8 : avk::kBf16x1;
  else p->var = vec_ok ? avk::kF32x4 : avk::kF32x1;
  p->vec = avk::variant_vec(p->var);
  p->nvec = V / p->vec;
  if ((long long)R * V >= (1LL << 46)) return AV_EUNSUPPORTED;
  return AV_OK;
}

// Chunks of the streaming backward: up to vecs_per_thread vectors per thread
// (raised as needed to keep <= 64 chunks per row).
int plan_chunks(const Plan& p, int vecs_per_thread, int* C) {
  if (vecs_per_thread < 0) return AV_EINVAL;
  const int nvmax = avk::variant_nvmax(p.var);
  const long long per_block = (long long)avk::kBlock * avk::kMaxChunks;
  const int nv_min = (int)((p.nvec + per_block - 1) / per_block);
  int nv = (vecs_per_thread == 0 || vecs_per_thread > nvmax) ? nvmax : vecs_per_thread;
  if (nv < nv_min) nv = nv_min;
  if (nv > nvmax) return AV_EUNSUPPORTED;
  const long long per_chunk = (long long)avk::kBlock * nv;
  *C = (int)((p.nvec + per_chunk - 1) / per_chunk);
  return AV_OK;
}

bool finite(float x) { return isfinite(x); }

// Temperature constants of the kernels: 1 / T and log2(e) / T, each the
// float32 rounding of the float64 value.
struct Temp {
  bool tm;
  float inv_t, inv_tl;
};
bool temperature_ok(float t, Temp* out) {
  if (!(t > 0.0f) || !finite(t)) return false;
  out->tm = t != 1.0f;
  out->inv_t = (float)(1.0 / (double)t);
  out->inv_tl = (float)(1.4426950408889634074 / (double)t);
  return true;
}

}  // namespace

extern "C" {

const char* av_status_str(int status) {
  switch (status) {
    case AV_OK: return "AV_OK";
    case AV_EINVAL: return "AV_EINVAL: invalid argument";
    case AV_EUNSUPPORTED: return "AV_EUNSUPPORTED: outside the implemented range";
    case AV_EHIP: return "AV_EHIP: HIP runtime error";
    default: return "unknown av_status";
  }
}

const char* av_last_hip_error(void) { return g_hip_err; }

size_t av_workspace_bytes(int B, int k, int R) {
  if (B < 1 || k < 1 || k > AV_MAX_K || R < 1 || (long long)R > (long long)B * k) return 0;
  return avk::ws_total(B, R);
}

int av_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < avk::kCtlBytes || !aligned16(workspace)) return AV_EINVAL;
  hipError_t e = avk::launch_zero((uint64_t*)workspace, workspace_bytes / 8, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

int av_length_head(const float* h, const float* w, float bias, float gamma, int B, int H, int k,
                   int round_mode, float* rate_out, int32_t* bk_out, void* stream) {
  if (!h || !w || !bk_out) return AV_EINVAL;
  if (B < 1 || H < 1 || k < 1 || k > AV_MAX_K) return AV_EINVAL;
  if (round_mode != AV_ROUND_CEIL && round_mode != AV_ROUND_FLOOR) return AV_EINVAL;
  if (!finite(bias) || !finite(gamma) || gamma < 0.0f) return AV_EINVAL;
  avk::HeadArgs a;
  a.h = h;
  a.w = w;
  a.rate = rate_out;
  a.bk = bk_out;
  a.bias = bias;
  a.gamma = gamma;
  a.B = B;
  a.H = H;
  a.k = k;
  a.mode = round_mode;
  hipError_t e = avk::launch_head(a, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

size_t av_head_update_workspace_bytes(int B) {
  if (B < 1) return 0;
  return (size_t)B * 2 * sizeof(double);
}

int av_length_head_update(const float* h, const int32_t* acc, const int32_t* bk, int B, int H, int k,
                          float* w, float* bias, float* m_w, float* v_w, float* m_b, float* v_b,
                          int step, double lr, double beta1, double beta2, double eps,
                          double weight_decay, float* loss_out, float* rate_out, float* grad_h_out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!h || !acc || !bk || !w || !bias || !m_w || !v_w || !m_b || !v_b || !workspace) return AV_EINVAL;
  if (B < 1 || H < 1 || k < 1 || k > AV_MAX_K || step < 1) return AV_EINVAL;
  if (!(isfinite(lr) && lr >= 0.0) || !(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0))
    return AV_EINVAL;
  if (!(isfinite(eps) && eps > 0.0) || !(isfinite(weight_decay) && weight_decay >= 0.0)) return AV_EINVAL;
  if (workspace_bytes < av_head_update_workspace_bytes(B) || ((uintptr_t)workspace & 7u) != 0) return AV_EINVAL;
  avk::HeadUpdArgs a;
  a.h = h;
  a.acc = acc;
  a.bk = bk;
  a.w = w;
  a.bias = bias;
  a.m_w = m_w;
  a.v_w = v_w;
  a.m_b = m_b;
  a.v_b = v_b;
  a.loss = loss_out;
  a.rate = rate_out;
  a.grad_h = grad_h_out;
  a.ws = (double*)workspace;
  a.B = B;
  a.H = H;
  a.k = k;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.wd = weight_decay;
  a.bc1 = 1.0 - pow(beta1, (double)step);
  a.sqrt_bc2 = sqrt(1.0 - pow(beta2, (double)step));
  hipError_t e = avk::launch_head_update(a, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

size_t av_spec_workspace_bytes(int B, int R) {
  if (B < 1 || R < 1) return 0;
  return (size_t)R * 16 + (size_t)B * avk::kSpecMaxChunks * 16;
}

int av_spec_verify(int dtype, int B, int k, int V, int R, const int32_t* row_off, const void* zp,
                   const void* zq, const int32_t* draft, const int32_t* bk, const float* u,
                   uint64_t seed, const float* row_stats_in, int stats_stride, int32_t* acc_len,
                   int32_t* token, float* row_stats, int32_t* status, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!zp || !zq || !draft || !u || !acc_len || !token || !workspace) return AV_EINVAL;
  if (!row_off && !bk) return AV_EINVAL;
  if (row_stats_in && stats_stride < 2) return AV_EINVAL;
  Plan p;
  int rc = plan_rows(dtype, B, k, V, R, row_off, zp, zq, nullptr, &p);
  if (rc != AV_OK) return rc;
  if (workspace_bytes < av_spec_workspace_bytes(B, R) || !aligned16(workspace)) return AV_EINVAL;
  // chunks of the race: at least kSpecChunkVecs vectors, at most kSpecMaxChunks per row
  int chunk = avk::kSpecChunkVecs;
  if ((long long)chunk * avk::kSpecMaxChunks < p.nvec)
    chunk = (p.nvec + avk::kSpecMaxChunks - 1) / avk::kSpecMaxChunks;
  const int nchunk = (p.nvec + chunk - 1) / chunk;
  avk::SpecArgs a;
  a.zp = zp;
  a.zq = zq;
  a.draft = draft;
  a.bk = bk;
  a.row_off = row_off;
  a.u = u;
  a.acc = acc_len;
  a.token = token;
  a.stats = row_stats;
  a.stats_in = row_stats_in;
  a.stats_stride = stats_stride;
  a.status = status;
  a.ws = (uint32_t*)workspace;
  a.chunks = (uint32_t*)((char*)workspace + (size_t)R * 16);
  a.chunk = chunk;
  a.nchunk = nchunk;
  a.seed = seed;
  a.B = B;
  a.k = k;
  a.V = V;
  a.R = R;
  a.nvec = p.nvec;
  a.ragged = p.ragged ? 1 : 0;
  hipError_t e = avk::launch_spec(p.var, a, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// The fused pass with its launch form chosen by the caller: onchip_limit as
// av_test_verify_opd_fwd, split 0 = automatic, 1 = whole rows, 2 = split rows,
// 3 = split tail (ragged only; half the rows whole, the rest in halves).
int verify_opd_fwd_impl(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                        const void* zp, const void* zq, const int32_t* draft, const int32_t* bk,
                        float lambda, float tau, float grad_scale, float temperature,
                        int32_t* tgt_argmax, int32_t* acc_len, float* row_loss, float* req_loss,
                        float* total_loss, float* row_stats, float* lse_q1, void* grad_zq,
                        int grad_dtype, int32_t* status, void* workspace, size_t workspace_bytes,
                        int onchip_limit, int split_mode, void* stream) {
  if (!zp || !zq || !draft || !tgt_argmax || !acc_len || !row_loss || !workspace) return AV_EINVAL;
  if (!row_off && !bk) return AV_EINVAL;
  if (!(lambda >= 0.0f && lambda <= 1.0f)) return AV_EINVAL;
  if (!(tau > 0.0f)) return AV_EINVAL;
  if (!finite(grad_scale)) return AV_EINVAL;
  Temp tp;
  if (!temperature_ok(temperature, &tp)) return AV_EINVAL;
  if (row_stats && !aligned16(row_stats)) return AV_EINVAL;
  if (!aligned16(workspace)) return AV_EINVAL;
  if (grad_zq && grad_dtype != AV_F32 && grad_dtype != AV_BF16) return AV_EUNSUPPORTED;
  Plan p;
  int rc = plan_rows(dtype, B, k, V, R, row_off, zp, zq, grad_zq, &p);
  if (rc != AV_OK) return rc;
  if (onchip_limit < 0 || split_mode < 0 || split_mode > 4) return AV_EINVAL;
  if (p.ragged && B + 1 > 4096) return AV_EUNSUPPORTED;  // offsets are cached in LDS
  if (workspace_bytes < avk::ws_total(B, R)) return AV_EINVAL;

  // Split rows: each verified row's halves on two CUs (both halves on chip,
  // no logit read twice where a whole row would not fit).  As the only form
  // of a launch (split_mode 2, on request only) it is slower than whole rows
  // on every workload measured (B=128 x 16 rows of 151936, ragged 605 rows of
  // 151936, 64 x 32 rows of 262144): the two statistics exchanges per row and
  // the per-row fixed costs are paid twice.  It pays where whole rows would
  // leave CUs idle: a ragged launch whose rows end in a partial round runs
  // the full rounds as whole rows and the rest as halves (split 3, chosen
  // automatically), and so does a dense launch with so few rows that their
  // halves fit one round (split 2, chosen automatically).  The halves meet at
  // a 64-vector boundary (1 KB of bfloat16 logits) near the middle of the row.
  const bool wide = p.var == avk::kBf16x8 || p.var == avk::kF32x4;
  int pv0 = (((p.nvec + 1) / 2) + 63) & ~63;
  if (pv0 >= p.nvec) pv0 = (p.nvec + 1) / 2;
  const long long part = p.nvec - pv0;  // the smaller half
  const long long slot = avk::kRowBlock;
  const int nl_max = avk::variant_row_lds(p.var);
  const int nr_row = avk::variant_row_regs(p.var);
  int nr_max = nr_row;

  const DeviceInfo* dev = nullptr;
  hipError_t e = device_info(&dev);
  if (e != hipSuccess) return hip_fail(e);

  // Dynamic LDS: ragged row offsets, or the longest-first schedule of the
  // dense layout (b_k as bytes and request indices as 16-bit words).
  const bool lpt = !p.ragged && B <= avk::kMaxLptRequests;
  size_t lds = 0;
  if (p.ragged) lds = (size_t)(B + 1) * sizeof(int32_t);
  else if (lpt) lds = (((size_t)B + 7) & ~(size_t)7) + (((size_t)B * 2 + 3) & ~(size_t)3);
  if (lds > kMaxDynLds) return AV_EUNSUPPORTED;
  const bool gb = grad_zq && grad_dtype == AV_BF16;
  auto occ_of = [&](bool full, int split, int nr) {
    return dev->occ[p.var][form_index(full, split, nr)][gb ? 1 : 0][tp.tm ? 1 : 0];
  };
  // The fast form needs every on-chip slot filled (in each half, when split)
  // and the default on-chip split.
  const bool row_full = onchip_limit == 0 && p.nvec >= (long long)(nr_row + nl_max) * slot;

  int split = 1, nwhole = 0;
  if (wide && p.nvec >= 4 && split_mode == 4) {
    split = 4;
  } else if (wide && p.nvec >= 2 && split_mode == 2) {
    split = 2;
  } else if (wide && p.nvec >= 2 && p.ragged && split_mode == 3) {
    split = 3;  // test form: the first half of the rows whole, the rest in halves
    nwhole = R / 2;
  } else if (wide && p.ragged && split_mode == 0 && row_full &&
             part >= (long long)(avk::kPairRegs + nl_max) * slot) {
    // Split tail: the rows of a last, partial round go in halves when their
    // halves fill at most one round (otherwise that round would take longer
    // than the whole rows it replaces).  Only for rows long enough that both
    // the rows and their halves fill the fast form's on-chip slots: shorter
    // rows are dominated by per-row fixed costs, which halves pay twice.
    const long long grid3 = (long long)occ_of(row_full, 3, nr_row) * dev->cus;
    if (grid3 >= 2) {
      const long long rem = R % grid3;
      if (rem > 0 && 2 * rem <= grid3) {
        split = 3;
        nwhole = (int)(R - rem);
      }
    }
  } else if (wide && !p.ragged && split_mode == 0 && row_full && 4LL * R <= (long long)dev->cus) {
    // A dense launch whose rows, in quarters, fit one round with a CU each:
    // every row in quarters.
    split = 4;
  } else if (wide && !p.ragged && split_mode == 0 && row_full &&
             part >= (long long)(avk::kPairRegs + nl_max) * slot && 2LL * R <= (long long)dev->cus) {
    // A dense launch whose rows, in halves, fit one round with a CU each (a
    // single request): every row in halves.  Measured on one request of 16
    // rows of 151936 bfloat16 logits (9 verified): 37.5 against 53.6 us.
    split = 2;
  }
  if (split == 2 && onchip_limit == 0 && part < (long long)(nr_max + nl_max) * slot &&
      part >= (long long)(avk::kPairRegs + nl_max) * slot)
    nr_max = avk::kPairRegs;  // fast form with fewer register slots
  if (split == 4) nr_max = avk::kPairRegs;  // quarters: 5 register slots (4.6 slots at V = 151936 bf16)
  int nr = nr_max, nl = nl_max;
  if (onchip_limit > 0) {
    nr = onchip_limit & 0xff;
    nl = (onchip_limit >> 8) & 0xff;
    if (nr > nr_max) nr = nr_max;
    if (nl > nl_max) nl = nl_max;
  }
  // split 3 in the fast form needs both the rows and their halves full
  const long long rowvecs = split == 2 ? part : split == 4 ? p.nvec / 4 : p.nvec;
  bool full = onchip_limit == 0 && rowvecs >= (long long)(nr_max + nl_max) * slot;
  if (split == 3 && part < (long long)(avk::kPairRegs + nl_max) * slot) full = false;
  if (split == 4) full = false;  // quarters: general form only
  const int occ = occ_of(full, split, nr_max);
  if (occ < 1) return AV_EUNSUPPORTED;
  long long grid = (long long)occ * dev->cus;
  if (split == 2 || split == 4) {
    // teams of co-resident workgroups; no more teams than rows
    if (grid > (long long)split * R) grid = (long long)split * R;
    grid -= grid % split;
    if (grid < split) return AV_EUNSUPPORTED;
  } else {
    const long long items = split == 3 ? 2LL * R - nwhole : (long long)R;
    if (grid > items) grid = items;
  }

  char* ws = (char*)workspace;
  avk::FwdArgs a;
  a.zp = zp;
  a.zq = zq;
  a.draft = draft;
  a.bk = bk;
  a.row_off = row_off;
  a.tgt = tgt_argmax;
  a.acc = acc_len;
  a.row_loss = row_loss;
  a.req_loss = req_loss;
  a.total = total_loss;
  a.stats = row_stats;
  a.lse1 = lse_q1;
  a.grad = grad_zq;
  a.status_out = status;
  a.ctl = (uint64_t*)ws;
  a.rowres = (uint64_t*)(ws + avk::ws_rowres_off());
  a.reqres = (uint64_t*)(ws + avk::ws_reqres_off(R));
  a.arrive = (uint64_t*)(ws + avk::ws_arrive_off(B, R));
  a.halfres = (uint64_t*)(ws + avk::ws_halfres_off(B, R));
  a.harrive = (uint64_t*)(ws + avk::ws_harrive_off(B, R));
  a.xres = (uint64_t*)(ws + avk::ws_xres_off(B, R));
  a.timeout_ticks = dev->ticks_per_ms * 2000;  // 2 s per wait
  a.B = B;
  a.k = k;
  a.V = V;
  a.R = R;
  a.nvec = p.nvec;
  a.nr = nr;
  a.nl = nl;
  a.ragged = p.ragged ? 1 : 0;
  a.lpt = lpt ? 1 : 0;
  a.split = split;
  a.pv0 = split > 1 ? pv0 : 0;
  a.nwhole = nwhole;
  // The last unverified rows of a longest-first launch go in quarters, so
  // that its last items are short: one round of the device's workgroups.
  a.nquart = (split == 1 && lpt && full) ? (int)grid : 0;
  a.gbf16 = gb ? 1 : 0;
  a.tm = tp.tm ? 1 : 0;
  a.lam = lambda;
  a.tau = tau;
  a.gs = grad_scale;
  a.inv_t = tp.inv_t;
  a.inv_tl = tp.inv_tl;
  e = avk::launch_fused(p.var, full, nr_max, a, (int)grid, lds, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int av_verify_opd_fwd(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                      const void* zp, const void* zq, const int32_t* draft, const int32_t* bk,
                      float lambda, float tau, float grad_scale, float temperature,
                      int32_t* tgt_argmax, int32_t* acc_len, float* row_loss, float* req_loss,
                      float* total_loss, float* row_stats, float* lse_q1, void* grad_zq,
                      int grad_dtype, int32_t* status, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return verify_opd_fwd_impl(dtype, B, k, V, R, row_off, zp, zq, draft, bk, lambda, tau, grad_scale,
                             temperature, tgt_argmax, acc_len, row_loss, req_loss, total_loss, row_stats,
                             lse_q1, grad_zq, grad_dtype, status, workspace, workspace_bytes, 0, 0, stream);
}

int av_init(void) {
  void* p = nullptr;
  hipError_t e = scratch_ptr(&p);
  const DeviceInfo* d = nullptr;
  if (e == hipSuccess) e = device_info(&d);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

size_t av_noalloc_max_bytes(void) { return AV_NOALLOC_SCRATCH_BYTES; }

int av_verify_opd_fwd_noalloc(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                              const void* zp, const void* zq, const int32_t* draft, const int32_t* bk,
                              float lambda, float tau, float grad_scale, float temperature,
                              int32_t* tgt_argmax, int32_t* acc_len, float* row_loss, float* req_loss,
                              float* total_loss, float* row_stats, float* lse_q1, void* grad_zq,
                              int grad_dtype, int32_t* status, void* stream) {
  const size_t need = av_workspace_bytes(B, k, R);
  if (need == 0) return AV_EINVAL;
  if (need > AV_NOALLOC_SCRATCH_BYTES) return AV_EUNSUPPORTED;
  void* ws = nullptr;
  hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return hip_fail(e);
  return verify_opd_fwd_impl(dtype, B, k, V, R, row_off, zp, zq, draft, bk, lambda, tau, grad_scale,
                             temperature, tgt_argmax, acc_len, row_loss, req_loss, total_loss, row_stats,
                             lse_q1, grad_zq, grad_dtype, status, ws, AV_NOALLOC_SCRATCH_BYTES, 0, 0, stream);
}

int av_test_verify_opd_fwd(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                           const void* zp, const void* zq, const int32_t* draft, const int32_t* bk,
                           float lambda, float tau, float grad_scale, float temperature,
                           int32_t* tgt_argmax, int32_t* acc_len, float* row_loss, float* req_loss,
                           float* total_loss, float* row_stats, float* lse_q1, void* grad_zq,
                           int grad_dtype, int32_t* status, void* workspace, size_t workspace_bytes,
                           int onchip_limit, int split_rows, void* stream) {
  return verify_opd_fwd_impl(dtype, B, k, V, R, row_off, zp, zq, draft, bk, lambda, tau, grad_scale,
                             temperature, tgt_argmax, acc_len, row_loss, req_loss, total_loss, row_stats,
                             lse_q1, grad_zq, grad_dtype, status, workspace, workspace_bytes, onchip_limit,
                             split_rows, stream);
}

int av_verify_opd_bwd(int dtype, int B, int k, int V, int R, const int32_t* row_off,
                      const void* zp, const void* zq, const int32_t* bk,
                      const int32_t* tgt_argmax, const float* row_stats, const float* lse_q1,
                      float lambda, float tau, float grad_scale, float temperature, void* grad_zq,
                      int grad_dtype, int vecs_per_thread, void* stream) {
  if (!zp || !zq || !tgt_argmax || !row_stats || !grad_zq) return AV_EINVAL;
  if (!row_off && !bk) return AV_EINVAL;
  if (!(lambda >= 0.0f && lambda <= 1.0f)) return AV_EINVAL;
  if (!(tau > 0.0f)) return AV_EINVAL;
  if (!finite(grad_scale)) return AV_EINVAL;
  Temp tp;
  if (!temperature_ok(temperature, &tp)) return AV_EINVAL;
  if (tp.tm && !lse_q1) return AV_EINVAL;
  if (!aligned16(row_stats)) return AV_EINVAL;
  if (grad_dtype != AV_F32 && grad_dtype != AV_BF16) return AV_EUNSUPPORTED;
  Plan p;
  int rc = plan_rows(dtype, B, k, V, R, row_off, zp, zq, grad_zq, &p);
  if (rc != AV_OK) return rc;
  int C = 0;
  rc = plan_chunks(p, vecs_per_thread, &C);
  if (rc != AV_OK) return rc;
  if ((long long)R * C > 0x7fffffffLL) return AV_EUNSUPPORTED;
  avk::BwdArgs a;
  a.zp = zp;
  a.zq = zq;
  a.bk = bk;
  a.tgt = tgt_argmax;
  a.stats = row_stats;
  a.lse1 = lse_q1;
  a.grad = grad_zq;
  a.B = B;
  a.k = k;
  a.V = V;
  a.R = R;
  a.C = C;
  a.nvec = p.nvec;
  a.ragged = p.ragged ? 1 : 0;
  a.gbf16 = grad_dtype == AV_BF16 ? 1 : 0;
  a.tm = tp.tm ? 1 : 0;
  a.lam = lambda;
  a.tau = tau;
  a.gs = grad_scale;
  a.inv_t = tp.inv_t;
  a.inv_tl = tp.inv_tl;
  hipError_t e = avk::launch_bwd(p.var, a, (hipStream_t)stream);
  return e == hipSuccess ? AV_OK : hip_fail(e);
}

}  // extern "C"
