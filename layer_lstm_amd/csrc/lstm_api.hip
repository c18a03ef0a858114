// lstm_api.hip -- the extern "C" entry points declared in include/lstm.h:
// argument checks, the work partition and workspace layout, and the launch
// sequence of each pass.  No device memory is allocated here.
#include <hip/hip_runtime.h>
#include <string.h>

#include <vector>

#include "internal.hpp"
#include "lstm.h"

namespace lstm {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LSTM_ERR_DEVICE;
  static int cached_dev = -1, cached_cus = 0, cached_ok = 0;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LSTM_ERR_DEVICE;
    cached_ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    cached_cus = prop.multiProcessorCount;
    cached_dev = dev;
  }
  if (!cached_ok) return LSTM_ERR_DEVICE;
  *cus = cached_cus;
  return LSTM_OK;
}

int make_plan(int64_t T, int64_t B, int64_t I, int64_t H, int dtype, Plan* p) {
  if (T < 0 || B < 0 || I < 0 || H <= 0) return LSTM_ERR_DIMS;
  if (dtype != LSTM_F32 && dtype != LSTM_BF16) return LSTM_ERR_DTYPE;
  if (H > 2048 || I > 65536 || T > ((int64_t)1 << 30)) return LSTM_ERR_UNSUPPORTED;
  if (T > 0 && B > 0 && T * B > ((int64_t)1 << 31) / (4 * H)) return LSTM_ERR_UNSUPPORTED;
  if (B * H >= ((int64_t)1 << 27)) return LSTM_ERR_UNSUPPORTED;  // per-step buffer offsets fit 31 bits
  int cus = 0;
  const int dev = device_cus(&cus);
  if (dev != LSTM_OK) return dev;

  memset(p, 0, sizeof(*p));
  p->T = T; p->B = B; p->I = I; p->H = H; p->dtype = dtype;
  p->esize = dtype ? 2 : 4;
  p->TB = T * B; p->G4 = 4 * H; p->Z = H + I;
  const int e = p->esize;
  const int KB = dtype ? 32 : 16;                       // MFMA k-block (elements)
  // H padded to a power of two, at least one k-block per wave
  int Hp = 4 * KB;
  while (Hp < H) Hp *= 2;
  p->Hp = Hp;

  p->cus = cus;
  p->nxcd = (cus % 32 == 0 && cus >= 32) ? cus / 32 : 1;

  // Partition of the persistent kernels.  Every work-group reads NB*H
  // values of h (forward) and NB*4H gate deltas (backward) per step, so the
  // fewest batch rows per group that still fit the grid come first, then
  // the most work-groups, then 4 waves before 8 (8 waves -- bf16 only -- hold
  // twice the W_h slice).  A first pass takes only partitions whose batch
  // groups divide evenly over the XCDs, so that each group's exchange stays
  // in one XCD's L2.  Fewer than 16 rows leave part of the 16-row MFMA batch
  // tile empty, which costs little next to the exchange.
  const int nb_opts[5] = {4, 8, 16, 32, 64};
  const int nj_opts[3] = {8, 16, 32};
  const int nw_opts[2] = {4, 8};
  bool found = false;
  for (int pass = 0; pass < 2 && !found; ++pass) {
    for (int a = 0; a < 5 && !found; ++a) {
      for (int c = 0; c < 3 && !found; ++c) {
        for (int d = 0; d < 2 && !found; ++d) {
          const int NB = nb_opts[a], NJ = nj_opts[c], NW = nw_opts[d];
          if (NW == 8 && !dtype) continue;
          const int64_t nBG = B > 0 ? (B + NB - 1) / NB : 1;
          const int64_t nJG = (H + NJ - 1) / NJ;
          if (nBG * nJG > cus) continue;
          if (pass == 0 && !(p->nxcd > 1 && nBG % p->nxcd == 0)) continue;
          const int NBr = NB < 16 ? 16 : NB;
          // forward: NJ/4 M-tiles of 16 interleaved gate rows in groups of
          // MW, the waves of a group splitting k; two tiles per wave when k
          // splits far enough (the same W_h values per wave either way)
          const int MTf = NJ / 4;
          if (MTf > NW) continue;
          const int MW = (MTf % 2 == 0 && Hp / ((2 * NW / MTf) * KB) >= 1) ? 2 : 1;
          const int KS = NW * MW / MTf;
          const int nkbw = Hp / (KS * KB);
          if (nkbw < 1 || MW * nkbw > 32) continue;
          const bool fdma = (H * e) % 1024 == 0;
          // h_{t-1}, partial tiles; direct-to-LDS path: two P buffers and
          // the record staging area
          size_t lds_f = (size_t)NBr * (Hp * e + 16) + (size_t)MTf * (KS - 1) * (NBr / 16) * 1024;
          if (fdma) lds_f += (size_t)2 * NB * NJ * 16 + (size_t)NB * (5 * NJ * e + 4 * NJ + 48);
          if (lds_f > 160 * 1024) continue;
          // the W_h slice is gathered through LDS at the start (recurrent.hip)
          const size_t lds_fw = lds_f < kColStageLds ? kColStageLds : lds_f;
          // backward: the VALU kernel (fp32, 4-row groups, <= 128 resident
          // W_h values per lane) or the MFMA kernel: 16-unit tiles of W_h^T,
          // the waves splitting the 4H gate rows
          const int vnct = Hp <= kRecThreads ? 1 : Hp / kRecThreads;
          const bool valu = !dtype && NB == 4 && NW == 4 && ((NJ == 8 && vnct <= 4) || (NJ == 16 && vnct == 1));
          const int MTb = NJ < 16 ? 1 : NJ / 16;
          const int nkb = Hp * e / (16 * NW);
          size_t lds_b;
          if (valu) {
            lds_b = (size_t)NBr * (4 * NJ * e + 16) + 4096 + (size_t)NB * NJ * 16;
          } else {
            if (nkb < 1 || MTb * nkb > 32 || NB * NJ > 1024) continue;
            // wave partials, db sums (1024 elements at most)
            lds_b = (size_t)NW * NBr * (16 * MTb + 4) * 4 + 16384;
            if (lds_b < kColStageLds) lds_b = kColStageLds;
          }
          p->NB = NB; p->NJ = NJ; p->nBG = (int)nBG; p->nJG = (int)nJG; p->grid = (int)(nBG * nJG);
          p->waves = NW;
          p->fwd_nkbw = nkbw;
          p->fwd_mw = MW;
          p->fwd_dma = fdma ? 1 : 0;
          p->bwd_valu = valu ? 1 : 0;
          p->bwd_mt = MTb;
          p->bwd_nkb = nkb;
          p->lds_fwd = lds_fw;
          p->lds_bwd = lds_b;
          found = true;
        }
      }
    }
  }
  if (!found) return LSTM_ERR_UNSUPPORTED;
  p->Bp = p->nBG * p->NB;
  {
    const int64_t fw = (int64_t)p->NB * (dtype ? Hp / 2 : Hp);         // forward words per work-group
    const int64_t bw = (int64_t)p->nJG * p->NB * p->NJ;                // backward words per work-group
    const int64_t mx = fw > bw ? fw : bw;
    p->words_per_thread = (int)((mx + 255) / 256);
  }
  // the gate-delta ring holds whole 16-row tiles per batch group
  const int64_t ring_rows = (int64_t)p->nBG * (p->NB < 16 ? 16 : p->NB);
  if (2 * ring_rows * 4 * Hp * e >= ((int64_t)1 << 30)) return LSTM_ERR_UNSUPPORTED;

  p->max_splits = 8;
  p->xcd_local = p->nxcd > 1 && p->nBG % p->nxcd == 0;

  const size_t HW = dtype ? (size_t)p->Hp / 2 : (size_t)p->Hp;
  // HX: tagged words [2][Bp][HW] (VALU forward), or packed h [2][Bp][Hp] +
  // flags [nBG][nJG]; PX: tagged words [2][nBG][nJG][Hp][NB] (VALU
  // backward), or gate deltas in 16-row tiles [2][nBG][max(NB,16)][4Hp] +
  // flags [nBG][nJG]
  p->off_hflags = align256(2 * (size_t)p->Bp * p->Hp * e);
  p->off_pflags = align256(2 * (size_t)ring_rows * 4 * p->Hp * e);
  const size_t nflag = align256((size_t)p->nBG * p->nJG * 4);
  size_t hx = p->off_hflags + nflag, px = p->off_pflags + nflag;
  if (fwd_vec_ok(*p) && hx < 2 * (size_t)p->Bp * HW * 8) hx = 2 * (size_t)p->Bp * HW * 8;
  if (p->bwd_valu && px < 2 * (size_t)p->nJG * p->Hp * p->Bp * 8) px = 2 * (size_t)p->nJG * p->Hp * p->Bp * 8;
  size_t off = 0;
  p->off_ctrl = off; off += 256;
  p->off_HX = off; p->bytes_HX = align256(hx); off += p->bytes_HX;
  p->off_PX = off; p->bytes_PX = align256(px); off += p->bytes_PX;
  p->off_P = off; off += align256((size_t)p->TB * p->G4 * 4);
  p->off_G = off; off += align256((size_t)p->TB * p->G4 * e);
  p->off_C = off; off += align256((size_t)p->TB * H * 4);
  p->off_gp = off; off += align256(gemm_partial_bytes(*p, cus));
  p->off_dbp = off; off += align256((size_t)p->nBG * p->G4 * 4);
  p->total = off;
  return LSTM_OK;
}

static int status_of(hipError_t e) {
  if (e == hipSuccess) return LSTM_OK;
  if (e == hipErrorCooperativeLaunchTooLarge) return LSTM_ERR_COOP;
  return LSTM_ERR_LAUNCH;
}

static bool misaligned(const void* ptr, int esize) { return ptr && ((uintptr_t)ptr % (uintptr_t)esize) != 0; }

// ---- per-kernel event timing (lstm_timing_enable / lstm_timing_read) ----
enum { kKinds = 7 };
struct Pending { int kind; hipEvent_t a, b; };
static bool g_timing_on = false;
static std::vector<Pending> g_pending;
static std::vector<hipEvent_t> g_pool;
static double g_total_ms[kKinds];
static uint64_t* g_stamps_fwd = nullptr;
static uint64_t* g_stamps_bwd = nullptr;
static size_t g_stamps_bytes = 0;
static int64_t g_launches[kKinds];

static hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets the launches made during its lifetime with two events.
struct Timed {
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr;
  Timed(int k, hipStream_t st) : kind(k), s(st) {
    if (g_timing_on && (a = take_event()) != nullptr && hipEventRecord(a, s) != hipSuccess) {
      g_pool.push_back(a);
      a = nullptr;
    }
  }
  ~Timed() {
    if (!a) return;
    hipEvent_t b = take_event();
    if (b && hipEventRecord(b, s) == hipSuccess) {
      g_pending.push_back({kind, a, b});
    } else {
      g_pool.push_back(a);
      if (b) g_pool.push_back(b);
    }
  }
};

// the stamp buffer holds [2 passes][kStampWGs][T][kPhases] clock values
static bool stamps_fit(const Plan& p) {
  return g_stamps_fwd && (size_t)2 * kStampWGs * p.T * kPhases * sizeof(uint64_t) <= g_stamps_bytes;
}

static void flush_timing() {
  for (const Pending& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_total_ms[p.kind] += ms;
      g_launches[p.kind] += 1;
    }
    g_pool.push_back(p.a);
    g_pool.push_back(p.b);
  }
  g_pending.clear();
}

}  // namespace lstm

using namespace lstm;

extern "C" {

int lstm_abi_version(void) { return LSTM_ABI_VERSION; }

const char* lstm_status_string(int status) {
  switch (status) {
    case LSTM_OK: return "ok";
    case LSTM_ERR_NULL: return "a required pointer is NULL";
    case LSTM_ERR_DIMS: return "invalid dimensions (T, B, I < 0 or H <= 0)";
    case LSTM_ERR_DTYPE: return "unsupported dtype";
    case LSTM_ERR_ALIGN: return "misaligned pointer";
    case LSTM_ERR_WORKSPACE: return "workspace too small";
    case LSTM_ERR_UNSUPPORTED: return "shape outside the supported envelope";
    case LSTM_ERR_COOP: return "persistent grid cannot be co-resident";
    case LSTM_ERR_LAUNCH: return "HIP launch failed";
    case LSTM_ERR_TIMEOUT: return "a recurrent step wait timed out";
    case LSTM_ERR_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
  }
}

int lstm_query(const lstm_shape* shape, size_t* workspace_bytes) {
  if (!shape || !workspace_bytes) return LSTM_ERR_NULL;
  if ((shape->flags & ~(LSTM_REVERSE | LSTM_GATES_IJFO | LSTM_TWO_BIAS)) != 0) return LSTM_ERR_DTYPE;
  Plan p;
  const int rc = make_plan(shape->T, shape->B, shape->I, shape->H, shape->dtype, &p);
  if (rc != LSTM_OK) return rc;
  *workspace_bytes = p.total;
  return LSTM_OK;
}

int lstm_query_plan(const lstm_shape* shape, lstm_plan_info* info) {
  if (!shape || !info) return LSTM_ERR_NULL;
  if ((shape->flags & ~(LSTM_REVERSE | LSTM_GATES_IJFO | LSTM_TWO_BIAS)) != 0) return LSTM_ERR_DTYPE;
  Plan p;
  const int rc = make_plan(shape->T, shape->B, shape->I, shape->H, shape->dtype, &p);
  if (rc != LSTM_OK) return rc;
  memset(info, 0, sizeof(*info));
  info->rows_per_group = p.NB;
  info->units_per_group = p.NJ;
  info->groups = p.nBG;
  info->units_groups = p.nJG;
  info->grid = p.grid;
  info->waves = p.waves;
  info->xcd_local = p.xcd_local ? 1 : 0;
  info->fwd_valu = fwd_vec_ok(p) ? 1 : 0;
  info->bwd_valu = p.bwd_valu ? 1 : 0;
  info->inproj_tiles_per_wg = inproj_tiles_per_wg(p);
  return LSTM_OK;
}

int lstm_fwd_train(const lstm_shape* shape, const void* x, const void* W, const void* b, const void* h0,
                   const void* c0, void* y, void* hT, void* cT, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!shape) return LSTM_ERR_NULL;
  if ((shape->flags & ~(LSTM_REVERSE | LSTM_GATES_IJFO | LSTM_TWO_BIAS)) != 0) return LSTM_ERR_DTYPE;
  Plan p;
  int rc = make_plan(shape->T, shape->B, shape->I, shape->H, shape->dtype, &p);
  if (rc != LSTM_OK) return rc;
  p.rev = (shape->flags & LSTM_REVERSE) ? 1 : 0;
  p.ijfo = (shape->flags & LSTM_GATES_IJFO) ? 1 : 0;
  p.two_bias = (shape->flags & LSTM_TWO_BIAS) ? 1 : 0;
  const int e = p.esize;
  if (!W || !workspace) return LSTM_ERR_NULL;
  if (p.TB * p.I > 0 && !x) return LSTM_ERR_NULL;
  if (p.TB > 0 && !y) return LSTM_ERR_NULL;
  if (p.B > 0 && (!hT || !cT)) return LSTM_ERR_NULL;
  if (misaligned(x, e) || misaligned(W, e) || misaligned(b, e) || misaligned(h0, e) || misaligned(c0, e) ||
      misaligned(y, e) || misaligned(hT, e) || misaligned(cT, e) || ((uintptr_t)workspace & 255u))
    return LSTM_ERR_ALIGN;
  if (workspace_bytes < p.total) return LSTM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t err = hipSuccess;

  if (p.B == 0) return LSTM_OK;
  if (p.T == 0) {
    Timed tm(6, s);
    err = launch_copy_state(h0, hT, (size_t)(p.B * p.H), e, s);
    if (err == hipSuccess) err = launch_copy_state(c0, cT, (size_t)(p.B * p.H), e, s);
    return status_of(err);
  }
  // the input projection's launch also clears the error word and both
  // step-exchange buffers (tags 0) for the recurrences that follow
  float* P = (float*)(ws + p.off_P);
  {
    Timed tm(0, s);
    err = launch_gemm_inproj(p, x, W, b, P, (float*)(ws + p.off_gp), ws + p.off_ctrl,
                             p.off_PX + p.bytes_PX - p.off_ctrl, s);
  }
  if (err == hipSuccess) {
    Timed tm(1, s);
    err = launch_fwd_recurrent(p, P, W, h0, c0, y, hT, cT, ws + p.off_G, (float*)(ws + p.off_C),
                               (uint64_t*)(ws + p.off_HX), (uint32_t*)(ws + p.off_ctrl),
                               stamps_fit(p) ? g_stamps_fwd : nullptr, s);
  }
  return status_of(err);
}

int lstm_bwd(const lstm_shape* shape, const void* dy, const void* dhT, const void* dcT, const void* x,
             const void* W, const void* h0, const void* c0, const void* y, void* workspace, size_t workspace_bytes,
             void* dx, void* dW, void* db, void* dh0, void* dc0, void* stream) {
  if (!shape) return LSTM_ERR_NULL;
  if ((shape->flags & ~(LSTM_REVERSE | LSTM_GATES_IJFO | LSTM_TWO_BIAS)) != 0) return LSTM_ERR_DTYPE;
  Plan p;
  int rc = make_plan(shape->T, shape->B, shape->I, shape->H, shape->dtype, &p);
  if (rc != LSTM_OK) return rc;
  p.rev = (shape->flags & LSTM_REVERSE) ? 1 : 0;
  p.ijfo = (shape->flags & LSTM_GATES_IJFO) ? 1 : 0;
  p.two_bias = (shape->flags & LSTM_TWO_BIAS) ? 1 : 0;
  const int e = p.esize;
  if (!W || !dW || !workspace) return LSTM_ERR_NULL;
  if (p.TB > 0 && (!dy || !y)) return LSTM_ERR_NULL;
  if (p.TB * p.I > 0 && (!x || !dx)) return LSTM_ERR_NULL;
  if (p.B > 0 && (!dh0 || !dc0)) return LSTM_ERR_NULL;
  if (misaligned(dy, e) || misaligned(dhT, e) || misaligned(dcT, e) || misaligned(x, e) || misaligned(W, e) ||
      misaligned(h0, e) || misaligned(c0, e) || misaligned(y, e) || misaligned(dx, e) || misaligned(dW, e) ||
      misaligned(db, e) || misaligned(dh0, e) || misaligned(dc0, e) || ((uintptr_t)workspace & 255u))
    return LSTM_ERR_ALIGN;
  if (workspace_bytes < p.total) return LSTM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t err = hipSuccess;

  if (p.T == 0 || p.B == 0) {
    Timed tm(6, s);
    err = launch_fill_zero(dW, (size_t)(p.G4 * p.Z) * e, s);
    if (err == hipSuccess && db) err = launch_fill_zero(db, (size_t)p.G4 * e, s);
    if (err == hipSuccess && p.B > 0) err = launch_copy_state(dhT, dh0, (size_t)(p.B * p.H), e, s);
    if (err == hipSuccess && p.B > 0) err = launch_copy_state(dcT, dc0, (size_t)(p.B * p.H), e, s);
    return status_of(err);
  }
  // The backward exchange buffer starts cleared: the forward clears it, and
  // every backward clears it again once its recurrence is done (in the dW
  // launch), so that a repeated backward finds it clean too.
  void* dG = ws + p.off_P;  // the input projection is dead after the forward
  {
    Timed tm(2, s);
    err = launch_bwd_recurrent(p, W, c0, dy, dhT, dcT, ws + p.off_G, (const float*)(ws + p.off_C), dG,
                               (uint64_t*)(ws + p.off_PX), db ? (float*)(ws + p.off_dbp) : nullptr, dh0, dc0,
                               (uint32_t*)(ws + p.off_ctrl),
                               stamps_fit(p) ? g_stamps_bwd : nullptr, s);
  }
  if (err == hipSuccess) {
    Timed tm(3, s);
    err = launch_gemm_dw(p, dG, x, h0, y, dW, (float*)(ws + p.off_gp), ws + p.off_PX, p.bytes_PX,
                         (const float*)(ws + p.off_dbp), db, s);
  }
  if (err == hipSuccess && p.I > 0) {
    Timed tm(4, s);
    err = launch_gemm_dx(p, dG, W, dx, (float*)(ws + p.off_gp), nullptr, 0, s);
  }
  return status_of(err);
}

int lstm_check_workspace(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return LSTM_ERR_NULL;
  if (workspace_bytes < 256) return LSTM_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return LSTM_ERR_LAUNCH;
  uint32_t word = 0;
  if (hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return LSTM_ERR_LAUNCH;
  if (word & kErrTimeout) {
    const uint32_t zero = 0;
    if (hipMemcpy(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return LSTM_ERR_LAUNCH;
    return LSTM_ERR_TIMEOUT;
  }
  return LSTM_OK;
}

int lstm_timing_enable(int on) {
  flush_timing();
  g_timing_on = on != 0;
  if (g_timing_on)
    for (int k = 0; k < kKinds; ++k) {
      g_total_ms[k] = 0.0;
      g_launches[k] = 0;
    }
  return LSTM_OK;
}

int lstm_stamps_set(void* device_buffer, size_t bytes, int64_t T) {
  if (!device_buffer || bytes == 0) {
    g_stamps_fwd = g_stamps_bwd = nullptr;
    g_stamps_bytes = 0;
    return LSTM_OK;
  }
  if (T <= 0) return LSTM_ERR_DIMS;
  if ((uintptr_t)device_buffer & 7u) return LSTM_ERR_ALIGN;
  const size_t half = (size_t)kStampWGs * T * kPhases * sizeof(uint64_t);
  if (bytes < 2 * half) return LSTM_ERR_WORKSPACE;
  g_stamps_fwd = (uint64_t*)device_buffer;
  g_stamps_bwd = (uint64_t*)((char*)device_buffer + half);
  g_stamps_bytes = bytes;
  return LSTM_OK;
}

int lstm_timing_read(int kind, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return LSTM_ERR_NULL;
  if (kind < 0 || kind >= kKinds) return LSTM_ERR_DIMS;
  flush_timing();
  *total_ms = g_total_ms[kind];
  *launches = g_launches[kind];
  return LSTM_OK;
}

}  // extern "C"
