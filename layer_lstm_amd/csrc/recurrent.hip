// recurrent.hip -- persistent forward and backward recurrences (gfx950).
//
// Forward ("SingleLayerLstmGrad" page, forward table): for t = 0..T-1
//   a_t = P_t + W_h h_{t-1}      (P_t = W_x x_t + b from the input projection)
//   i,f,o = sigmoid, g = tanh;   c_t = f c_{t-1} + i g;   h_t = o tanh(c_t)
// Backward (same page, "反向传播算法" steps 1-6): for t = T-1..0
//   dh = dy_t + dh_carry;  dc = dh o (1 - tanh^2 c_t) + dc_carry
//   do = dh tanh(c_t) o(1-o); dg = dc i (1-g^2); di = dc g i(1-i);
//   df = dc c_{t-1} f(1-f);  dc_carry = dc f;  dh_carry = W_h^T dG_t
// with dh_carry/dc_carry starting from dhT/dcT, and dh0/dc0 the carries
// left after t = 0.
//
// One launch per direction of time; the grid (nBG x nJG work-groups, one
// per CU, all resident at once) runs every step.  Work-group
// (bg, jg) owns batch rows [bg*NB, +NB) and hidden units [jg*NJ, +NJ); it
// keeps the 4*NJ rows of W_h that belong to its units (gates i,f,g,o of each
// unit) in VGPRs as MFMA fragments for the whole launch.  Batch groups never
// talk to each other: rows of the batch are independent in both passes.
//
// Rows are interleaved: MFMA row 4u + g is gate g of unit u, so one lane
// holds the four gates of one (unit, batch) pair after each product and the
// cell update needs no data movement.
//
// Exchange per step inside a batch group, through tagged 8-byte words
// (value + step tag, relaxed agent-scope atomics; see device_common.hpp):
//   forward:  h_t of the group's rows (each work-group writes its units);
//   backward: each work-group writes the fp32 partial product
//             W_h[rows of its units]^T dG_t for all H columns, and every
//             work-group sums, in a fixed order, the partials of its own
//             units from all work-groups of the group.  The words of one
//             batch group are contiguous ([group][producer][unit][row]),
//             so a reader fetches only lines that it uses.
// No other grid-wide synchronisation is used.  A thread issues all of its
// exchange loads of a round at once (up to C in flight) and re-polls only
// the words whose tag is not there yet, so a step costs about one memory
// round trip of waiting, not one per word.
//
// Compile-time shapes (H is padded to Hp, a power of two): NKBW k-blocks of
// W_h per wave in the forward, MTW 16-column tiles of W_h^T per wave and
// NKBR k-blocks of the 4*NJ rows in the backward; NBT 16-row batch tiles.
#include "device_common.hpp"
#include "internal.hpp"

namespace lstm {

constexpr int kWaves = 4;                 // waves per work-group
constexpr int kRecThreads = 64 * kWaves;

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
  uint64_t* HX;     // [2][Bp][HW] exchange words
  uint32_t* err;
  uint64_t* stamps; // optional [kStampWGs][T][kPhases] clock stamps
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp, HW;
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
  uint64_t* PX;     // [2][nBG][nJG][Hp][NB] exchange words (fp32 partials)
  float* DBP;       // [nBG][4H] per-batch-group db partials, interleaved gates
  void* dh0;
  void* dc0;
  uint32_t* err;
  uint64_t* stamps;
  int T, B, H, Z, NB, NJ, nJG, Hp, Bp;
};

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
  if (dead) return;
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
      return;
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
      if ((pending >> c) & 1u) wv[c] = xload(base + off[c]);
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

// ---------------------------------------------------------------------------
template <typename T, int NBT, int NKBW, int C>
__global__ void __launch_bounds__(kRecThreads, 1) fwd_rec_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int bg = blockIdx.x / a.nJG, jg = blockIdx.x % a.nJG;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int MT = a.NJ / 4;                   // M-tiles (16 interleaved gate rows = 4 units)
  const int KS = kWaves / MT;                // waves splitting k per M-tile
  const int mt = w / KS, wk = w % KS;        // this wave's M-tile and k part
  const int kb0 = wk * NKBW;
  const int strideH = a.Hp * E + 16;         // LDS row of h_{t-1}
  const int NBr = a.NB < 16 ? 16 : a.NB;     // rows of the batch tiles (rows >= NB stay zero)
  char* Hl = smem;                           // [NBr][strideH]
  float* red = (float*)(smem + NBr * strideH);  // [MT*(KS-1) partial slots][NBT][64][4]
  const int64_t G4 = 4 * (int64_t)a.H;
  const int u = j0 + 4 * mt + fq;            // unit of this lane's elementwise results
  bool dead = false;

  // --- resident W_h fragments: rows 16*mt + fr (gate fr&3 of unit 4*mt + fr/4)
  u32x4_t wreg[NKBW];
  {
    const int ur = j0 + 4 * mt + (fr >> 2), g = fr & 3;
    const T* wrow = (const T*)a.W + ((int64_t)g * a.H + ur) * a.Z;
#pragma unroll
    for (int i = 0; i < NKBW; ++i) {
      T tmp[16 / E];
      const int k = (kb0 + i) * KB + fq * (16 / E);
#pragma unroll
      for (int e = 0; e < 16 / E; ++e) tmp[e] = (ur < a.H && k + e < a.H) ? wrow[k + e] : T(0);
      wreg[i] = __builtin_bit_cast(u32x4_t, tmp);
    }
  }
  const int NBv = (a.B - b0) < a.NB ? (a.B - b0) : a.NB;  // valid rows of this group
  // --- zero the padding of h_{t-1} in LDS once (k >= H, rows past the group or B)
  for (int idx = tid; idx < NBr * a.Hp; idx += kRecThreads) {
    const int bl = idx / a.Hp, k = idx % a.Hp;
    if (k >= a.H || bl >= NBv) *(T*)(Hl + bl * strideH + k * E) = T(0);
  }
  // --- cell state of this lane's elements (wk == 0 waves own the elementwise)
  float cst[NBT];
#pragma unroll
  for (int nt = 0; nt < NBT; ++nt) {
    const int b = b0 + 16 * nt + fr;
    cst[nt] = (a.c0 && u < a.H && 16 * nt + fr < NBv) ? ldf<T>(a.c0, (int64_t)b * a.H + u) : 0.f;
  }
  constexpr int vpw = (E == 2) ? 2 : 1;                  // values per exchange word
  const int HWv = (a.H + vpw - 1) / vpw;                 // words per row carrying data
  const int lgHW = 31 - __builtin_clz(a.HW);             // HW is a power of two
  const int total = NBv << lgHW;                         // exchange words read per step
  const uint32_t doff = (uint32_t)(tid % total);         // target of unused load slots

  // The input projection of this lane's elements is prefetched one step
  // ahead (at the end of the previous step), so that no wait of a step on its
  // exchange words or its product also waits for this load.
  f32x4_t pf[NBT];
  auto load_p = [&](int tt) {
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt) {
      const int b = b0 + 16 * nt + fr;
      pf[nt] = (wk == 0 && tt < a.T && u < a.H && 16 * nt + fr < NBv)
                   ? *(const f32x4_t*)(a.P + ((int64_t)tt * a.B + b) * G4 + 4 * (int64_t)u)
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_p(0);

  for (int t = 0; t < a.T; ++t) {
    stamp(a.stamps, a.T, t, 0);
    // h_{t-1} words: word idx = bl * HW + kw of this group's rows (HW a power
    // of two); slots past the data point at a harmless word of the group
    const uint64_t* src = a.HX + ((int64_t)((t - 1) & 1) * a.Bp + b0) * a.HW;
    uint32_t off[C];
    uint32_t live = 0;
    uint64_t wv[C];
    if (t > 0) {
      live = plan_h_round<C>(off, 0, tid, total, a.HW - 1, HWv, doff);
      issue_tagged<C>(wv, src, off);
    }
    __syncthreads();  // previous step's readers of Hl are done
    // h_{t-1} -> LDS
    if (t == 0) {
      for (int idx = tid; idx < NBv * a.H; idx += kRecThreads) {
        const int bl = idx / a.H, k = idx % a.H;
        const T v = a.h0 ? ((const T*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : T(0);
        *(T*)(Hl + bl * strideH + k * E) = v;
      }
    } else {
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)t, a.err, dead);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          if ((live >> c) & 1u) {
            const int bl = off[c] >> lgHW, kw = off[c] & (a.HW - 1);
            *(uint32_t*)(Hl + bl * strideH + kw * 4) = (uint32_t)wv[c];  // one fp32 or two bf16
          }
        }
        base += kRecThreads * C;
        if (base >= total) break;
        live = plan_h_round<C>(off, base, tid, total, a.HW - 1, HWv, doff);
        issue_tagged<C>(wv, src, off);
      }
    }
    stamp(a.stamps, a.T, t, 1);
    __syncthreads();
    stamp(a.stamps, a.T, t, 2);

    // MFMA: acc[nt] = W_h[rows of M-tile mt, k part] . h_{t-1}[tile nt]^T,
    // with CH independent accumulator chains per tile (summed in a fixed order)
    constexpr int CH = NBT == 1 ? (NKBW >= 4 ? 4 : NKBW) : (NBT == 2 && NKBW >= 2 ? 2 : 1);
    f32x4_t acc[NBT], part[NBT][CH];
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt)
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) part[nt][ch] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const char* hb0 = Hl + fr * strideH + kb0 * 64 + fq * 16;
#pragma unroll
    for (int i = 0; i < NKBW; ++i) {
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        const u32x4_t hb = *(const u32x4_t*)(hb0 + 16 * nt * strideH + i * 64);
        part[nt][i % CH] = Mfma<T>::mac(wreg[i], hb, part[nt][i % CH]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt) {
      acc[nt] = part[nt][0];
#pragma unroll
      for (int ch = 1; ch < CH; ++ch) acc[nt] += part[nt][ch];
    }
    stamp(a.stamps, a.T, t, 3);
    if (KS > 1) {
      if (wk != 0) {
#pragma unroll
        for (int nt = 0; nt < NBT; ++nt)
          *(f32x4_t*)(red + (((mt * (KS - 1) + wk - 1) * NBT + nt) * 64 + lane) * 4) = acc[nt];
      }
      __syncthreads();
      if (wk == 0) {
        for (int k2 = 1; k2 < KS; ++k2) {
#pragma unroll
          for (int nt = 0; nt < NBT; ++nt)
            acc[nt] += *(const f32x4_t*)(red + (((mt * (KS - 1) + k2 - 1) * NBT + nt) * 64 + lane) * 4);
        }
      }
    }

    stamp(a.stamps, a.T, t, 4);
    // elementwise: gates, cell, hidden; outputs and the exchange word
    if (wk == 0) {
      uint64_t* dst = a.HX + (int64_t)(t & 1) * a.Bp * a.HW;
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        const int b = b0 + 16 * nt + fr;
        const bool valid = u < a.H && 16 * nt + fr < NBv;
        const f32x4_t z = acc[nt] + pf[nt];
        const float ig = sigmoidf(z[0]), fg = sigmoidf(z[1]), gg = tanh_f(z[2]), og = sigmoidf(z[3]);
        const float c = fg * cst[nt] + ig * gg;
        const float h = og * tanh_f(c);
        cst[nt] = c;
        const T hq = Elem<T>::from_f(h);
        if constexpr (E == 2) {
          // pack units u (even lane group) and u+1 (next lane group) into one word
          const uint32_t mine = (uint32_t)__builtin_bit_cast(uint16_t, hq);
          const uint32_t next = (uint32_t)__shfl_down((int)mine, 16, 64);
          if ((fq & 1) == 0 && valid) {
            const uint32_t both = mine | ((u + 1 < a.H) ? (next << 16) : 0u);
            __hip_atomic_store(dst + (int64_t)b * a.HW + u / 2, ((uint64_t)(t + 1) << 32) | both,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          if (valid) xstore(dst + (int64_t)b * a.HW + u, h, (uint32_t)(t + 1));
        }
        if (valid) {
          const int64_t o = (int64_t)t * a.B + b;
          ((T*)a.y)[o * a.H + u] = hq;
          T gq[4] = {Elem<T>::from_f(ig), Elem<T>::from_f(fg), Elem<T>::from_f(gg), Elem<T>::from_f(og)};
          if constexpr (E == 4)
            *(f32x4_t*)((T*)a.Gs + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(f32x4_t, gq);
          else
            *(uint64_t*)((T*)a.Gs + o * G4 + 4 * (int64_t)u) = __builtin_bit_cast(uint64_t, gq);
          a.Cs[o * a.H + u] = c;
          if (t == a.T - 1) {
            ((T*)a.hT)[(int64_t)b * a.H + u] = hq;
            ((T*)a.cT)[(int64_t)b * a.H + u] = Elem<T>::from_f(c);
          }
        }
      }
    }
    load_p(t + 1);
    stamp(a.stamps, a.T, t, 5);
  }
  // T == 0 is handled on the host
}

// ---------------------------------------------------------------------------
template <typename T, int NKBR, int MTW, int C>
__global__ void __launch_bounds__(kRecThreads, 1) bwd_rec_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  const int bg = blockIdx.x / a.nJG, jg = blockIdx.x % a.nJG;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int NBT = a.NB < 16 ? 1 : a.NB / 16;
  const int NBr = a.NB < 16 ? 16 : a.NB;     // rows of the batch tiles (rows >= NB stay zero)
  const int nel = a.NB * a.NJ;               // (batch row, unit) elements, a power of two
  const int lgNB = 31 - __builtin_clz(a.NB), lgNel = 31 - __builtin_clz(nel);
  const int EPT = nel > kRecThreads ? nel / kRecThreads : 1;  // elements per thread (1, 2 or 4)
  const int TPE = nel < kRecThreads ? kRecThreads / nel : 1;  // threads per element (1..8)
  const int strideD = 4 * a.NJ * E + 16;
  char* Dl = smem;                                     // [NBr][strideD] gate deltas (B operand)
  float* sums = (float*)(smem + NBr * strideD);        // [4][kRecThreads] gather sums
  float* dba = sums + 4 * kRecThreads;                 // [nel][4] db: gate deltas summed over time
  for (int idx = tid; idx < 4 * nel; idx += kRecThreads) dba[idx] = 0.f;
  for (int idx = tid; idx < NBr * strideD / 4; idx += kRecThreads) ((uint32_t*)Dl)[idx] = 0u;
  const int64_t G4 = 4 * (int64_t)a.H;
  const int gtotal = a.nJG * nel;                      // exchange words read per step
  const int nBG = a.Bp / a.NB;
  const int HpNB = a.Hp * a.NB;                        // words of one producer's block
  const uint32_t doff = (uint32_t)(tid % gtotal);      // target of unused load slots
  bool dead = false;

  // --- resident fragments of W_h^T: A[m = column k][kslot = row r], column
  // tile of fragment i is w + kWaves*i
  u32x4_t wreg[MTW * NKBR];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
#pragma unroll
    for (int kb = 0; kb < NKBR; ++kb) {
      const int k = 16 * (w + kWaves * i) + fr;  // column of W_h
      T tmp[16 / E];
#pragma unroll
      for (int e = 0; e < 16 / E; ++e) {
        const int r = kb * KB + fq * (16 / E) + e;  // interleaved row: unit r/4, gate r%4
        const int ur = j0 + (r >> 2), g = r & 3;
        tmp[e] = (k < a.H && ur < a.H) ? ((const T*)a.W)[((int64_t)g * a.H + ur) * a.Z + k] : T(0);
      }
      wreg[i * NKBR + kb] = __builtin_bit_cast(u32x4_t, tmp);
    }
  }

  // --- elementwise ownership: elements e = tid + 256*s (s < EPT), batch fastest
  float dcc[4], dhc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = tid + kRecThreads * s;
    const int b = b0 + (e & (a.NB - 1)), uu = j0 + (e >> lgNB);
    const bool valid = s < EPT && e < nel && b < a.B && uu < a.H;
    dcc[s] = (valid && a.dcT) ? ldf<T>(a.dcT, (int64_t)b * a.H + uu) : 0.f;
    dhc[s] = (valid && a.dhT) ? ldf<T>(a.dhT, (int64_t)b * a.H + uu) : 0.f;
  }

  // Elementwise operands of a step (activated gates, c_t, c_{t-1}, dy_t) are
  // prefetched one step ahead, at the end of the step before.
  float pg[4][4], pc[4], pcp[4], pdy[4];
  auto load_ops = [&](int tt) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = tid + kRecThreads * s;
      const int bl = e & (a.NB - 1), uu = j0 + (e >> lgNB);
      const int b = b0 + bl;
      pg[s][0] = pg[s][1] = pg[s][2] = pg[s][3] = 0.f;
      pc[s] = pcp[s] = pdy[s] = 0.f;
      if (tt >= 0 && s < EPT && e < nel && b < a.B && uu < a.H) {
        const int64_t o = (int64_t)tt * a.B + b;
        if constexpr (E == 4) {
          const f32x4_t gv = *(const f32x4_t*)((const T*)a.Gs + o * G4 + 4 * (int64_t)uu);
          pg[s][0] = gv[0]; pg[s][1] = gv[1]; pg[s][2] = gv[2]; pg[s][3] = gv[3];
        } else {
          const uint64_t raw = *(const uint64_t*)((const T*)a.Gs + o * G4 + 4 * (int64_t)uu);
          pg[s][0] = bf2f((bf16_t)raw); pg[s][1] = bf2f((bf16_t)(raw >> 16));
          pg[s][2] = bf2f((bf16_t)(raw >> 32)); pg[s][3] = bf2f((bf16_t)(raw >> 48));
        }
        pc[s] = a.Cs[o * a.H + uu];
        pcp[s] = tt > 0 ? a.Cs[(o - a.B) * a.H + uu] : (a.c0 ? ldf<T>(a.c0, (int64_t)b * a.H + uu) : 0.f);
        pdy[s] = ldf<T>(a.dy, o * a.H + uu);
      }
    }
  };
  load_ops(a.T - 1);

  for (int t = a.T - 1; t >= -1; --t) {
    const int step = a.T - 1 - (t < 0 ? 0 : t);
    if (t >= 0) stamp(a.stamps, a.T, step, 0);
    // 1. gather dh_carry: sum over work-groups of the partials produced at
    //    step t+1.  Word idx = jg' * nel + e (e = jj * NB + bl): a thread
    //    always meets the same element slot(s), in increasing jg' order, and
    //    the TPE threads sharing an element are then added in a fixed order.
    const bool gather = t < a.T - 1;
    const uint64_t* src = a.PX + ((int64_t)((t + 1) & 1) * nBG + bg) * a.nJG * HpNB;
    uint32_t off[C];
    uint32_t live = 0;
    uint64_t wv[C];
    if (gather) {
      live = plan_dh_round<C>(off, 0, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
      issue_tagged<C>(wv, src, off);
    }
    if (gather) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)(t + 2), a.err, dead);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float v = ((live >> c) & 1u) ? xval(wv[c]) : 0.f;
          const int slot = ((base / kRecThreads) + c) & (EPT - 1);
          acc[0] += slot == 0 ? v : 0.f;
          acc[1] += slot == 1 ? v : 0.f;
          acc[2] += slot == 2 ? v : 0.f;
          acc[3] += slot == 3 ? v : 0.f;
        }
        base += kRecThreads * C;
        if (base >= gtotal) break;
        live = plan_dh_round<C>(off, base, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
        issue_tagged<C>(wv, src, off);
      }
      // sums[s][tid] holds this thread's part of element tid + 256*s (EPT > 1),
      // or of element tid % nel (TPE > 1)
#pragma unroll
      for (int s = 0; s < 4; ++s) sums[kRecThreads * s + tid] = acc[s];
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = tid + kRecThreads * s;
        if (s < EPT && e < nel) {
          float v = 0.f;
          for (int q = 0; q < TPE; ++q) v += sums[kRecThreads * s + tid + q * nel];
          dhc[s] = v;
        }
      }
      __syncthreads();
    }
    if (t < 0) break;
    stamp(a.stamps, a.T, step, 1);

    // 2. gate deltas of this step
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = tid + kRecThreads * s;
      if (s < EPT && e < nel) {
        const int bl = e & (a.NB - 1), jj = e >> lgNB;
        const int b = b0 + bl, uu = j0 + jj;
        T dq[4] = {T(0), T(0), T(0), T(0)};
        if (b < a.B && uu < a.H) {
          const int64_t o = (int64_t)t * a.B + b;
          const float gi = pg[s][0], gf = pg[s][1], gg = pg[s][2], go = pg[s][3];
          const float c = pc[s], cprev = pcp[s];
          const float tc = tanh_f(c);
          const float dh = pdy[s] + dhc[s];
          const float dc = dh * go * (1.f - tc * tc) + dcc[s];
          const float d_o = dh * tc * go * (1.f - go);
          const float d_g = dc * gi * (1.f - gg * gg);
          const float d_i = dc * gg * gi * (1.f - gi);
          const float d_f = dc * cprev * gf * (1.f - gf);
          dcc[s] = dc * gf;
          *(f32x4_t*)(dba + 4 * e) += f32x4_t{d_i, d_f, d_g, d_o};
          dq[0] = Elem<T>::from_f(d_i); dq[1] = Elem<T>::from_f(d_f);
          dq[2] = Elem<T>::from_f(d_g); dq[3] = Elem<T>::from_f(d_o);
          if constexpr (E == 4)
            *(f32x4_t*)((T*)a.dG + o * G4 + 4 * (int64_t)uu) = __builtin_bit_cast(f32x4_t, dq);
          else
            *(uint64_t*)((T*)a.dG + o * G4 + 4 * (int64_t)uu) = __builtin_bit_cast(uint64_t, dq);
        }
        if constexpr (E == 4)
          *(f32x4_t*)(Dl + bl * strideD + jj * 16) = __builtin_bit_cast(f32x4_t, dq);
        else
          *(uint64_t*)(Dl + bl * strideD + jj * 8) = __builtin_bit_cast(uint64_t, dq);
      }
    }
    __syncthreads();
    stamp(a.stamps, a.T, step, 2);

    // 3. partial[k][b] = sum_{r in my rows} W_h[r][k] dG[b][r], all k < H
    uint64_t* dst = a.PX + (((int64_t)(t & 1) * nBG + bg) * a.nJG + jg) * HpNB;
    for (int nt = 0; nt < NBT; ++nt) {
      u32x4_t breg[NKBR];
#pragma unroll
      for (int kb = 0; kb < NKBR; ++kb)
        breg[kb] = *(const u32x4_t*)(Dl + (16 * nt + fr) * strideD + kb * 64 + fq * 16);
      const int bl = 16 * nt + fr, b = b0 + bl;
      const bool bvalid = bl < a.NB && b < a.B;
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKBR; ++kb) acc = Mfma<T>::mac(wreg[i * NKBR + kb], breg[kb], acc);
        if (bvalid) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 16 * (w + kWaves * i) + 4 * fq + e;
            if (k < a.H) xstore(dst + (int64_t)k * a.NB + bl, acc[e], (uint32_t)(t + 1));
          }
        }
      }
    }
    stamp(a.stamps, a.T, step, 3);
    load_ops(t - 1);
    stamp(a.stamps, a.T, step, 4);
    __syncthreads();  // Dl is rewritten next step
    stamp(a.stamps, a.T, step, 5);
  }

  // db partial of this work-group: for each (unit, gate), the sum over its
  // batch rows (in row order) of the per-element sums over time
  if (a.DBP) {
    __syncthreads();
    for (int r = tid; r < 4 * a.NJ; r += kRecThreads) {
      const int jj = r >> 2, g = r & 3;
      float v = 0.f;
      for (int bl = 0; bl < a.NB; ++bl) v += dba[4 * ((jj << lgNB) + bl) + g];
      if (j0 + jj < a.H) a.DBP[(int64_t)bg * G4 + 4 * (j0 + jj) + g] = v;
    }
  }

  // dh0 / dc0
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = tid + kRecThreads * s;
    const int b = b0 + (e & (a.NB - 1)), uu = j0 + (e >> lgNB);
    if (s < EPT && e < nel && b < a.B && uu < a.H) {
      ((T*)a.dh0)[(int64_t)b * a.H + uu] = Elem<T>::from_f(dhc[s]);
      ((T*)a.dc0)[(int64_t)b * a.H + uu] = Elem<T>::from_f(dcc[s]);
    }
  }
}

// ---------------------------------------------------------------------------
// The persistent kernels need every work-group of the grid resident at
// once.  The grid never exceeds the CU count and each work-group fits a CU
// on its own; the occupancy query confirms that the device can hold the
// whole grid before the kernel is dispatched as an ordinary launch (a
// cooperative launch would guarantee the same but costs about 15 us more per
// dispatch).  If other work holds CUs, the waiting work-groups spin until it
// drains; every wait is bounded (kWaitTicks) and reports LSTM_ERR_TIMEOUT.
template <typename K>
static hipError_t coop_launch(K kernel, int grid, size_t lds, void* arg, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  void* args[] = {arg};
  int per_cu = 0, dev = 0, cus = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kernel, kRecThreads, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if (per_cu < 1 || (int64_t)per_cu * cus < grid) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel((const void*)kernel, dim3(grid), dim3(kRecThreads), args, lds, s);
}

template <typename T, int NBT, int C>
static hipError_t fwd_dispatch_c(const Plan& p, FwdArgs& a, hipStream_t s) {
  switch (p.fwd_nkbw) {
    case 1: return coop_launch(fwd_rec_kernel<T, NBT, 1, C>, p.grid, p.lds_fwd, &a, s);
    case 2: return coop_launch(fwd_rec_kernel<T, NBT, 2, C>, p.grid, p.lds_fwd, &a, s);
    case 4: return coop_launch(fwd_rec_kernel<T, NBT, 4, C>, p.grid, p.lds_fwd, &a, s);
    case 8: return coop_launch(fwd_rec_kernel<T, NBT, 8, C>, p.grid, p.lds_fwd, &a, s);
    case 16: return coop_launch(fwd_rec_kernel<T, NBT, 16, C>, p.grid, p.lds_fwd, &a, s);
    case 32: return coop_launch(fwd_rec_kernel<T, NBT, 32, (C > 16 ? 16 : C)>, p.grid, p.lds_fwd, &a, s);
  }
  return hipErrorInvalidValue;
}

// exchange words in flight per thread: as many as a thread reads per step,
// so that few load slots go unused
template <typename T, int NBT>
static hipError_t fwd_dispatch(const Plan& p, FwdArgs& a, hipStream_t s) {
  if (p.words_per_thread <= 4) return fwd_dispatch_c<T, NBT, 4>(p, a, s);
  return fwd_dispatch_c<T, NBT, 16>(p, a, s);
}

hipError_t launch_fwd_recurrent(const Plan& p, const float* P, const void* W, const void* h0, const void* c0,
                                void* y, void* hT, void* cT, void* Gs, float* Cs, uint64_t* HX, uint32_t* err,
                                uint64_t* stamps, hipStream_t s) {
  FwdArgs a{P, W, h0, c0, y, hT, cT, Gs, Cs, HX, err, stamps, (int)p.T, (int)p.B, (int)p.H, (int)p.Z, p.NB, p.NJ,
            p.nJG, p.Hp, p.Bp, p.dtype ? (p.Hp / 2) : p.Hp};
  const int nbt = p.NB < 16 ? 1 : p.NB / 16;
  if (p.dtype) {
    if (nbt == 1) return fwd_dispatch<bf16_t, 1>(p, a, s);
    if (nbt == 2) return fwd_dispatch<bf16_t, 2>(p, a, s);
    if (nbt == 4) return fwd_dispatch<bf16_t, 4>(p, a, s);
  } else {
    if (nbt == 1) return fwd_dispatch<float, 1>(p, a, s);
    if (nbt == 2) return fwd_dispatch<float, 2>(p, a, s);
    if (nbt == 4) return fwd_dispatch<float, 4>(p, a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int NKBR, int C>
static hipError_t bwd_dispatch_c(const Plan& p, BwdArgs& a, hipStream_t s) {
  switch (p.bwd_mtw) {
    case 1: return coop_launch(bwd_rec_kernel<T, NKBR, 1, C>, p.grid, p.lds_bwd, &a, s);
    case 2: return coop_launch(bwd_rec_kernel<T, NKBR, 2, C>, p.grid, p.lds_bwd, &a, s);
    case 4: return coop_launch(bwd_rec_kernel<T, NKBR, 4, C>, p.grid, p.lds_bwd, &a, s);
    case 8:
      if constexpr (8 * NKBR <= 32) return coop_launch(bwd_rec_kernel<T, NKBR, 8, (8 * NKBR <= 8 ? C : (C > 16 ? 16 : C))>, p.grid, p.lds_bwd, &a, s);
      break;
    case 16:
      if constexpr (16 * NKBR <= 32) return coop_launch(bwd_rec_kernel<T, NKBR, 16, (C > 16 ? 16 : C)>, p.grid, p.lds_bwd, &a, s);
      break;
    case 32:
      if constexpr (32 * NKBR <= 32) return coop_launch(bwd_rec_kernel<T, NKBR, 32, (C > 8 ? 8 : C)>, p.grid, p.lds_bwd, &a, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int NKBR>
static hipError_t bwd_dispatch(const Plan& p, BwdArgs& a, hipStream_t s) {
  if (p.words_per_thread <= 4) return bwd_dispatch_c<T, NKBR, 4>(p, a, s);
  return bwd_dispatch_c<T, NKBR, 16>(p, a, s);
}

hipError_t launch_bwd_recurrent(const Plan& p, const void* W, const void* c0, const void* dy, const void* dhT,
                                const void* dcT, const void* Gs, const float* Cs, void* dG, uint64_t* PX, float* DBP,
                                void* dh0, void* dc0, uint32_t* err, uint64_t* stamps, hipStream_t s) {
  BwdArgs a{W, c0, dy, dhT, dcT, Gs, Cs, dG, PX, DBP, dh0, dc0, err, stamps, (int)p.T, (int)p.B, (int)p.H, (int)p.Z,
            p.NB, p.NJ, p.nJG, p.Hp, p.Bp};
  const int nkbr = 4 * p.NJ * p.esize / 64;
  if (p.dtype) {
    if (nkbr == 1) return bwd_dispatch<bf16_t, 1>(p, a, s);
    if (nkbr == 2) return bwd_dispatch<bf16_t, 2>(p, a, s);
  } else {
    if (nkbr == 2) return bwd_dispatch<float, 2>(p, a, s);
    if (nkbr == 4) return bwd_dispatch<float, 4>(p, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lstm
