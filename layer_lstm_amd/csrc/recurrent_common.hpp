// recurrent_common.hpp -- pieces shared by the persistent recurrent kernels
// (recurrent.hip: MFMA products; recurrent_vec.hip: VALU products for
// small batch groups): launch arguments, the work-group roles, the bounded
// tagged-word waits and the exchange round plans.
#pragma once
#include "device_common.hpp"
#include "internal.hpp"

namespace lstm {

struct FwdArgs {
  const float* P;   // [TB][4H] fp32, interleaved gates, bias included
  const void* W;    // [4H][H+I]
  const void* h0;   // [B][H] or null
  const void* c0;   // [B][H] or null
  void* y;          // [T][B][H]
  void* hT;         // [B][H]
  void* cT;         // [B][H]
  void* Gs;         // [TB][4H] activated gates, interleaved
  float* Cs;        // [TB][H] cell states
  uint64_t* HX;     // [2][Bp][HW] exchange words (tagged-word kernels)
  void* HD;         // [2][Bp][Hp] packed h ring (flag kernels), T elements
  uint32_t* HF;     // [nBG][nJG] step flags of the flag kernels
  uint32_t hd_bytes;
  uint32_t* err;
  uint64_t* stamps; // optional [kStampWGs][T][kPhases] clock stamps
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp, HW;
  int nBG, nxcd, local;
  int rev;          // 1: the reverse direction (steps run from t = T-1 down to 0)
  int ijfo;         // gate-block order of W (gate_block)
  uint32_t* claims;    // [grid] role claims (cleared before the launch) or null
  int fail_step, misplace;  // test hooks (Plan)
  const int32_t* len;  // [B] sequence lengths (the seq_length mask in its per-row form) or null
  const float* c0f;    // [B][H] fp32 initial cell state in place of c0 (a stack's chunk continuing the
                       // previous one from its fp32 record), or null
};

struct BwdArgs {
  const void* W;
  const void* c0;
  const void* dy;   // [T][B][H]
  const void* dhT;  // [B][H] or null
  const void* dcT;  // [B][H] or null
  const void* Gs;
  const float* Cs;
  void* dG;         // [TB][4H] gate deltas, interleaved
  uint64_t* PX;     // [2][nBG][nJG][Hp][NB] exchange words (fp32 partials; VALU kernel)
  void* GD;         // [2][nBG][16-row tiles] gate deltas in MFMA fragment order, T elements (MFMA kernel)
  uint32_t* GF;     // [nBG][nJG] step flags of the MFMA kernel
  uint32_t gd_bytes;
  float* DBP;       // [nBG][4H] per-batch-group db partials, interleaved gates
  void* dh0;
  void* dc0;
  uint32_t* err;
  uint64_t* stamps;
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp;
  int nBG, nxcd, local;
  int rev;          // 1: the reverse direction (the forward ran from t = T-1 down to 0)
  int ijfo;         // gate-block order of W (gate_block)
  uint32_t* claims;    // [grid] role claims or null (see FwdArgs)
  int fail_step, misplace;
  const int32_t* len;  // [B] sequence lengths or null (see FwdArgs)
  // a stack's chunk of steps: c_{t-1} of its first step from the fp32 record
  // (cprevf, in place of c0), and the carries in fp32 (carry: [2][B][H], dh
  // then dc) read at the start in place of dhT/dcT (carry_in) and written
  // at the end in place of dh0/dc0 (carry_out); each element's carries are
  // read and written by the one thread that owns it
  const float* cprevf;
  float* carry;
  int carry_in, carry_out;
};

// Several recurrences in one persistent launch (the two directions of a
// bidirectional layer, the layers of a stack's wave): slot k takes
// work-groups [k*grid1, (k+1)*grid1) and its own arguments.
constexpr int kMaxSlots = 4;
template <class A>
struct Launch {
  A s[kMaxSlots];
  int nslots;
  int grid1;  // work-groups per slot
};

// This work-group's slot arguments (a uniform choice among the kernel's
// arguments) and its index within the slot.
template <class A>
__device__ __forceinline__ int slot_select(const Launch<A>& L, A& a) {
  const int k = L.nslots > 1 ? (int)blockIdx.x / L.grid1 : 0;
  a = L.s[0];
#pragma unroll
  for (int j = 1; j < kMaxSlots; ++j)
    if (k == j) a = L.s[j];
  if (k > 0) a.stamps = nullptr;  // phase stamps come from the first slot only
  return (int)blockIdx.x - k * L.grid1;
}

// Work-groups of a recurrent launch: every slot's.
template <class A>
inline int launch_grid(const Plan& p, const Launch<A>& L) { return (L.nslots > 1 ? L.nslots : 1) * p.grid; }

// Length of sequence b (T when there are no lengths): steps at times
// t >= len_of(b) lie past its end.
__device__ __forceinline__ int len_of(const int32_t* len, int b, int T) { return len ? len[b] : T; }

// Time index in memory of processing step s (s = 0 is the step that reads
// the initial state): s itself, or T-1-s in the reverse direction.  Loops,
// exchange slots and flags count processing steps; every tensor indexed by
// time (P, y, the record, dy, the gate deltas) is addressed through this.
__device__ __forceinline__ int mem_t(int s, int T, int rev) { return rev ? T - 1 - s : s; }

// Phase stamps: thread 0 of the first kStampWGs work-groups records the
// 100 MHz real-time clock (s_memrealtime) at kPhases points of every step when
// a stamp buffer is given; slot layout [wg][step][phase], steps in execution
// order.
__device__ __forceinline__ void stamp(uint64_t* buf, int T, int step, int phase) {
  if (buf && threadIdx.x == 0 && blockIdx.x < kStampWGs)
    buf[((int64_t)blockIdx.x * T + step) * kPhases + phase] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ bool err_set(uint32_t* err) {
  return __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
}

// Role of work-group i of a direction: (batch group, unit group).  In the XCD-local
// layout, XCD x holds batch groups [x*nBG/nxcd, (x+1)*nBG/nxcd) whole.  The
// device deals the work-groups of a dispatch to its XCDs round robin from a
// starting XCD that varies between dispatches, so work-group i runs on XCD
// (s + i) % nxcd and i / nxcd numbers the work-groups of one XCD without
// repeats; the XCD itself is read from the hardware.  (Slot k of a launch
// of several recurrences starts at grid index k*grid1, a multiple of nxcd in
// this layout, so the same holds for its own indices.)  (Were the dealing
// ever different, two work-groups could take one role -- they would compute
// and write the same values -- and another role would stay empty, which
// the bounded waits report as a time-out; results are never mixed.)
// (misplace: a test hook -- work-group 0 takes the role its neighbouring XCD
// would give it, as a device that dealt differently would.)
__device__ __forceinline__ void take_role(int i, int nBG, int nJG, int nxcd, int local, int misplace, int& bg,
                                          int& jg) {
  if (!local) {
    bg = i / nJG;
    jg = i % nJG;
    return;
  }
  const uint32_t shift = (misplace && i == 0) ? 1u : 0u;
  const int x = (int)((xcc_id() + shift) % (uint32_t)nxcd), k = i / nxcd;
  bg = x * (nBG / nxcd) + k / nJG;
  jg = k % nJG;
}

// Claim role (bg, jg): a second claimant of one role means the layout's
// assumption about the dealing failed -- recorded as a time-out with the
// placement bit (the host then stops using the XCD-local layout).
__device__ __forceinline__ void claim_role(uint32_t* claims, int role, uint32_t* err) {
  if (claims && threadIdx.x == 0 && atomicAdd(claims + role, 1u) != 0u) atomicOr(err, kErrTimeout | kErrPlacement);
}

// Test hook (lstm_debug_inject): at step `fail_step` (in execution order),
// thread 0 of work-group 0 of each direction acts as if its wait had timed
// out -- the error word is set and its later waits return at once -- so
// that the time-out path runs with every kernel still exiting normally.
__device__ __forceinline__ void inject_failure(int fail_step, int step, int wg, uint32_t* err, bool& dead) {
  if (fail_step == step && wg == 0 && threadIdx.x == 0) {
    atomicOr(err, kErrTimeout);
    dead = true;
  }
}

// Tagged-word reads, in two halves so that independent loads can be issued
// between them: issue_tagged() sends the C loads of a thread at once;
// complete_tagged() waits until every wanted word (bit c of `live`) carries
// `tag`, re-polling all still-missing words once per round trip.  Loads
// retire in order, so anything issued after issue_tagged() does not delay
// the check.  The wait is bounded: past kWaitTicks (or once another thread
// has recorded an error) the error word is set and `dead` makes this and
// every later wait of the thread return at once.
template <int C>
__device__ __forceinline__ void issue_tagged(uint64_t (&wv)[C], const uint64_t* base, const uint32_t (&off)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) wv[c] = xload(base + off[c]);
}

template <int C>
__device__ __forceinline__ void complete_tagged(uint64_t (&wv)[C], const uint64_t* base, const uint32_t (&off)[C],
                                                uint32_t live, uint32_t tag, uint32_t* err, bool& dead) {
  if (dead) {
    wait_vmem();
    return;
  }
  uint64_t t0 = 0;
  uint32_t rounds = 0;
  while (true) {
    uint32_t pending = 0;
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (((live >> c) & 1u) && xtag(wv[c]) != tag) pending |= 1u << c;
    if (!pending) return;
    if (t0 == 0) {
      t0 = now_ticks();
    } else if ((++rounds & 15u) == 0 && (now_ticks() - t0 > kWaitTicks || err_set(err))) {
      atomicOr(err, kErrTimeout);
      dead = true;
      wait_vmem();
      return;
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
      if ((pending >> c) & 1u) wv[c] = xload(base + off[c]);
  }
}

// ---------------------------------------------------------------------------
// Flag exchange (the MFMA kernels): a producer writes its payload packed,
// waits until those stores have completed, and then sets its step flag; a
// consumer polls the flags of every producer it needs (one thread each) and
// then reads the payload with 16-byte loads.  Stores and loads are
// device-coherent (write-through stores, loads that do not hit a stale line)
// or, in the XCD-local layout, plain stores that stay in the shared L2 --
// the same pairing as the tagged words.
__device__ __forceinline__ void store_flag(uint32_t* f, uint32_t v, bool local) {
  if (local)
    *f = v;
  else
    __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait until *f >= want; false (and the error word set) past
// kWaitTicks or once another thread has recorded an error.
__device__ __forceinline__ bool wait_flag(const uint32_t* f, uint32_t want, uint32_t* err, bool& dead) {
  if (dead) return false;
  uint64_t t0 = 0;
  uint32_t rounds = 0;
  while (__hip_atomic_load(const_cast<uint32_t*>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
    if (t0 == 0) {
      t0 = now_ticks();
    } else if ((++rounds & 15u) == 0 && (now_ticks() - t0 > kWaitTicks || err_set(err))) {
      atomicOr(err, kErrTimeout);
      dead = true;
      return false;
    }
  }
  return true;
}

// 16 bytes at byte offset `off` of a buffer, read device-coherently (sc1).
__device__ __forceinline__ u32x4_t load16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Element store of a packed payload: plain in the XCD-local layout, else
// device-coherent.
template <typename T>
__device__ __forceinline__ void store_elem(T* p, T v, bool local) {
  if (local) {
    *p = v;
  } else if constexpr (sizeof(T) == 2) {
    __hip_atomic_store((uint16_t*)p, __builtin_bit_cast(uint16_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    __hip_atomic_store((uint32_t*)p, __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Forward round plan: word idx = base + c*256 + tid of the group's rows
// (idx = row * HW + word, HW a power of two); a word is wanted if it lies
// in [0, total) and carries data (word < HWv).  Unwanted slots point at
// `doff`, a word of the group, so that no two slots of a wave hit one line.
template <int C>
__device__ __forceinline__ uint32_t plan_h_round(uint32_t (&off)[C], int base, int tid, int total, int hw_mask,
                                                 int hwv, uint32_t doff) {
  uint32_t live = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int idx = base + c * kRecThreads + tid;
    const bool lv = idx < total && (idx & hw_mask) < hwv;
    off[c] = lv ? (uint32_t)idx : doff;
    live |= (lv ? 1u : 0u) << c;
  }
  return live;
}

// Backward round plan: word idx = jg' * nel + e, e = jj * NB + bl; the word
// is partial[jg'][unit j0 + jj][row bl] of the group's exchange block
// [nJG][Hp][NB], i.e. at jg' * Hp * NB + j0 * NB + e.
template <int C>
__device__ __forceinline__ uint32_t plan_dh_round(uint32_t (&off)[C], int base, int tid, int gtotal, int nel, int lg_nel,
                                                  int NB, int lg_nb, int j0, int b0, int B, int H, int HpNB,
                                                  uint32_t doff) {
  uint32_t live = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int idx = base + c * kRecThreads + tid;
    const int e = idx & (nel - 1), g2 = idx >> lg_nel;
    const int bl = e & (NB - 1), uu = j0 + (e >> lg_nb);
    const bool lv = idx < gtotal && b0 + bl < B && uu < H;
    off[c] = lv ? (uint32_t)g2 * (uint32_t)HpNB + (uint32_t)(j0 * NB + e) : doff;
    live |= (lv ? 1u : 0u) << c;
  }
  return live;
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  return Elem<T>::to_f(((const T*)p)[i]);
}

// Persistent launches of one device run one at a time, whatever stream the
// caller gives: two such grids resident together could each hold part of
// the CUs that the other's waiting work-groups need.  persistent_before(s)
// makes stream s wait for the last persistent launch of the current device
// when that was on another stream; persistent_after(s) records its end
// (one event per device, kept for the life of the process).
hipError_t persistent_before(hipStream_t s);
hipError_t persistent_after(hipStream_t s);
// creates the current device's ordering event ahead of the first launch
hipError_t persistent_prepare();

// The persistent kernels need every work-group of the grid resident at
// once.  The grid never exceeds the CU count and each work-group fits a CU
// on its own; the occupancy query confirms that the device can hold the
// whole grid before the kernel is dispatched as an ordinary launch (a
// cooperative launch would guarantee the same but costs about 15 us more per
// dispatch).  If other work holds CUs, the waiting work-groups spin until it
// drains; every wait is bounded (kWaitTicks) and reports LSTM_ERR_TIMEOUT.
// The LDS request is raised to at least kOneGroupLds, more than half a CU's
// LDS, so that two work-groups never share a CU (they would share its SIMDs
// and serialise each other's steps).
constexpr size_t kOneGroupLds = 82 * 1024;
template <typename K>
inline hipError_t coop_launch(K kernel, int grid, size_t lds, void* arg, hipStream_t s, int threads = kRecThreads) {
  if (lds < kOneGroupLds) lds = kOneGroupLds;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  void* args[] = {arg};
  int per_cu = 0, dev = 0, cus = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, threads, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu < 1 || (int64_t)per_cu * cus < grid) return hipErrorCooperativeLaunchTooLarge;
  if ((e = persistent_before(s)) != hipSuccess) return e;
  if ((e = hipLaunchKernel((const void*)kernel, dim3(grid), dim3(threads), args, lds, s)) != hipSuccess) return e;
  return persistent_after(s);
}

// v of another lane of the quad (DPP quad_perm control CTRL).
template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// VALU recurrences for fp32 batch groups of 4 rows (recurrent_vec.hip)
hipError_t launch_fwd_vec(const Plan& p, Launch<FwdArgs>& a, hipStream_t s);
hipError_t launch_bwd_vec(const Plan& p, Launch<BwdArgs>& a, hipStream_t s);
// MFMA backward, column partition (recurrent_bwd.hip)
hipError_t launch_bwd_col(const Plan& p, Launch<BwdArgs>& a, hipStream_t s);

}  // namespace lstm
