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
#include "recurrent_common.hpp"

namespace lstm {

// ---------------------------------------------------------------------------
template <typename T, int NBT, int NKBW, int C>
__global__ void __launch_bounds__(kRecThreads, 1) fwd_rec_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  int bg, jg;
  take_role(a.nBG, a.nJG, a.nxcd, a.local, bg, jg);
  const bool local = a.local != 0;
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
  // packed h ring: row b of slot s at byte ((s * Bp + b) * Hp) * E; the chunks
  // covering [0, H) of the group's valid rows are read each step
  const int rowB = a.Hp * E;                              // bytes per row
  const int cpr = (a.H * E + 15) / 16;                    // 16-byte chunks per row with data
  const int nchunk = NBv * cpr;
  const __amdgpu_buffer_rsrc_t hd_rsrc = make_rsrc(a.HD, a.hd_bytes);
  T* HDt = (T*)a.HD;

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
    // wait until every work-group of the batch group has published h_{t-1}
    if (t > 0 && tid < a.nJG) wait_flag(a.HF + bg * a.nJG + tid, (uint32_t)t, a.err, dead);
    __syncthreads();  // flags seen; the previous step's readers of Hl are done
    // h_{t-1} -> LDS
    if (t == 0) {
      wait_vmem();
      for (int idx = tid; idx < NBv * a.H; idx += kRecThreads) {
        const int bl = idx / a.H, k = idx % a.H;
        const T v = a.h0 ? ((const T*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : T(0);
        *(T*)(Hl + bl * strideH + k * E) = v;
      }
    } else {
      const uint32_t slot0 = (uint32_t)(((t - 1) & 1) * a.Bp + b0) * (uint32_t)rowB;
      for (int q0 = 0; q0 < nchunk; q0 += kRecThreads * C) {
        u32x4_t v[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int q = q0 + c * kRecThreads + tid;
          const int bl = q / cpr, cc = q - bl * cpr;
          v[c] = q < nchunk ? load16_coherent(hd_rsrc, slot0 + (uint32_t)(bl * rowB + cc * 16)) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int q = q0 + c * kRecThreads + tid;
          const int bl = q / cpr, cc = q - bl * cpr;
          if (q < nchunk) *(u32x4_t*)(Hl + bl * strideH + cc * 16) = v[c];
        }
      }
    }
    // Everything this wave issued before (last step's stores, the input
    // prefetch) has completed by now; saying so keeps the compiler from
    // waiting for stores before it reuses their registers below.
    wait_vmem();
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
    // elementwise: gates, cell, hidden; h_t is published first (stores, their
    // completion, then the flag), the other outputs after
    float gv[NBT][4], cv[NBT];
    T hv[NBT];
    if (wk == 0) {
      T* dst = HDt + (int64_t)(t & 1) * a.Bp * a.Hp;
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        const int b = b0 + 16 * nt + fr;
        const bool valid = u < a.H && 16 * nt + fr < NBv;
        const f32x4_t z = acc[nt] + pf[nt];
        gv[nt][0] = sigmoidf(z[0]);
        gv[nt][1] = sigmoidf(z[1]);
        gv[nt][2] = tanh_f(z[2]);
        gv[nt][3] = sigmoidf(z[3]);
        const float c = gv[nt][1] * cst[nt] + gv[nt][0] * gv[nt][2];
        const float h = gv[nt][3] * tanh_f(c);
        cst[nt] = c;
        cv[nt] = c;
        hv[nt] = Elem<T>::from_f(h);
        if (valid) store_elem<T>(dst + (int64_t)b * a.Hp + u, hv[nt], local);
      }
    }
    wait_vmem();
    __syncthreads();
    if (tid == 0) store_flag(a.HF + bg * a.nJG + jg, (uint32_t)(t + 1), local);
    if (wk == 0) {
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        const int b = b0 + 16 * nt + fr;
        const bool valid = u < a.H && 16 * nt + fr < NBv;
        const float ig = gv[nt][0], fg = gv[nt][1], gg = gv[nt][2], og = gv[nt][3];
        const float c = cv[nt];
        const T hq = hv[nt];
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
// VNCT > 0 selects the VALU form of the partial product (fp32, batch groups
// of 4 rows; a 16x16 MFMA tile would leave 12 of its 16 batch columns empty
// there): lane quad qd = t/4 owns the W_h columns 256*i + 4*qd + {0..3}
// (i < VNCT), lane p = t%4 of the quad the row chunk [p*VR/4, (p+1)*VR/4)
// of the VR = 4*NJ rows of the work-group's units, kept in VGPRs.  Each lane
// forms the 16 (column, batch row) pieces of its chunk with fp32 FMAs --
// one LDS value of dG feeds four columns -- and a reduce-scatter across the
// quad (DPP) leaves lane p with the four batch-row sums of column
// 256*i + 4*qd + p, stored as 32 contiguous bytes.
template <typename T, int NKBR, int MTW, int C, int VNCT = 0, int VR = 0>
__global__ void __launch_bounds__(kRecThreads, 1) bwd_rec_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 15, fq = lane >> 4;
  int bg, jg;
  take_role(a.nBG, a.nJG, a.nxcd, a.local, bg, jg);
  const bool local = a.local != 0;
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
  // flag exchange: 16-byte chunks (row, 4 units) of this work-group's units,
  // TPC threads per chunk (nel <= 1024, so the sums fit the 4 KB LDS area)
  const int nchk = nel / 4;
  const int tpc = nchk >= kRecThreads ? 1 : kRecThreads / nchk;
  const __amdgpu_buffer_rsrc_t pd_rsrc = make_rsrc(a.PD, a.pd_bytes);
  const int nBG = a.nBG;
  const int HpNB = a.Hp * a.NB;                        // words of one producer's block
  const uint32_t doff = (uint32_t)(tid % gtotal);      // target of unused load slots
  bool dead = false;

  // --- resident fragments of W_h^T: A[m = column k][kslot = row r], column
  // tile of fragment i is w + kWaves*i
  u32x4_t wreg[VNCT ? 1 : MTW * NKBR];
  constexpr int VRC = VNCT ? VR / 4 : 1;  // rows per quad lane
  float wq[VNCT ? VNCT : 1][4][VRC];
  const int qd = tid >> 2, qp = tid & 3;
  if constexpr (VNCT > 0) {
#pragma unroll
    for (int i = 0; i < VNCT; ++i)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int k = kRecThreads * i + 4 * qd + cc;
#pragma unroll
        for (int rr = 0; rr < VRC; ++rr) {
          const int r = qp * VRC + rr, ur = j0 + (r >> 2), g = r & 3;
          wq[i][cc][rr] = (k < a.H && ur < a.H) ? ldf<T>(a.W, ((int64_t)g * a.H + ur) * a.Z + k) : 0.f;
        }
      }
  }
  if constexpr (VNCT == 0)
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
  // (EPTM bounds EPT at compile time: batch groups of 4 rows have at most 64
  // elements per work-group)
  constexpr int EPTM = VNCT ? 1 : 4;
  float dcc[EPTM], dhc[EPTM];
#pragma unroll
  for (int s = 0; s < EPTM; ++s) {
    const int e = tid + kRecThreads * s;
    const int b = b0 + (e & (a.NB - 1)), uu = j0 + (e >> lgNB);
    const bool valid = s < EPT && e < nel && b < a.B && uu < a.H;
    dcc[s] = (valid && a.dcT) ? ldf<T>(a.dcT, (int64_t)b * a.H + uu) : 0.f;
    dhc[s] = (valid && a.dhT) ? ldf<T>(a.dhT, (int64_t)b * a.H + uu) : 0.f;
  }

  // Elementwise operands of a step (activated gates, c_t, c_{t-1}, dy_t) are
  // prefetched one step ahead, at the end of the step before.
  float pg[EPTM][4], pc[EPTM], pcp[EPTM], pdy[EPTM];
  bool own[EPTM];
  int64_t g_off[EPTM], c_off[EPTM];  // element offsets in Gs and in [B][H] tensors
#pragma unroll
  for (int s = 0; s < EPTM; ++s) {
    const int e = tid + kRecThreads * s;
    const int b = b0 + (e & (a.NB - 1)), uu = j0 + (e >> lgNB);
    own[s] = s < EPT && e < nel && b < a.B && uu < a.H;
    g_off[s] = (int64_t)b * G4 + 4 * (int64_t)uu;
    c_off[s] = (int64_t)b * a.H + uu;
  }
  const int64_t stepG = (int64_t)a.B * G4, stepC = (int64_t)a.B * a.H;
  auto load_ops = [&](int tt) {
    const int64_t oG = (int64_t)tt * stepG, oC = (int64_t)tt * stepC;
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
      pg[s][0] = pg[s][1] = pg[s][2] = pg[s][3] = 0.f;
      pc[s] = pcp[s] = pdy[s] = 0.f;
      if (tt >= 0 && own[s]) {
        if constexpr (E == 4) {
          const f32x4_t gv = *(const f32x4_t*)((const T*)a.Gs + oG + g_off[s]);
          pg[s][0] = gv[0]; pg[s][1] = gv[1]; pg[s][2] = gv[2]; pg[s][3] = gv[3];
        } else {
          const uint64_t raw = *(const uint64_t*)((const T*)a.Gs + oG + g_off[s]);
          pg[s][0] = bf2f((bf16_t)raw); pg[s][1] = bf2f((bf16_t)(raw >> 16));
          pg[s][2] = bf2f((bf16_t)(raw >> 32)); pg[s][3] = bf2f((bf16_t)(raw >> 48));
        }
        pc[s] = a.Cs[oC + c_off[s]];
        pcp[s] = tt > 0 ? a.Cs[oC - stepC + c_off[s]] : (a.c0 ? ldf<T>(a.c0, c_off[s]) : 0.f);
        pdy[s] = ldf<T>(a.dy, oC + c_off[s]);
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
    if (!gather) wait_vmem();
    if constexpr (VNCT == 0) {
      // Flag exchange: the partials of step t+1 sit packed as [producer][row
      // bl][column k] fp32; the NB*NJ/4 16-byte chunks (bl, 4 units) of this
      // work-group's units are summed over producers jg' = r, r+TPC, ... by
      // the TPC threads of a chunk, then over r in LDS, in that fixed order.
      if (gather) {
        if (tid < a.nJG) wait_flag(a.PF + bg * a.nJG + tid, (uint32_t)(a.T - t - 1), a.err, dead);
        __syncthreads();
        const uint32_t base0 = (uint32_t)((((t + 1) & 1) * nBG + bg) * a.nJG) * (uint32_t)(a.NB * a.Hp * 4);
        const uint32_t pstride = (uint32_t)(a.NB * a.Hp * 4);  // bytes per producer block
        for (int qq = tid; qq < tpc * nchk; qq += kRecThreads) {
          const int q = qq % nchk, r = qq / nchk;     // chunk, producer residue
          const int bl = q / (a.NJ / 4), jq = q % (a.NJ / 4);
          const uint32_t off0 = base0 + (uint32_t)((bl * a.Hp + j0 + 4 * jq) * 4);
          f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
          for (int g0 = r; g0 < a.nJG; g0 += tpc * C) {
            u32x4_t v[C];
#pragma unroll
            for (int c = 0; c < C; ++c) {
              const int g2 = g0 + c * tpc;
              v[c] = g2 < a.nJG ? load16_coherent(pd_rsrc, off0 + (uint32_t)g2 * pstride) : u32x4_t{0, 0, 0, 0};
            }
#pragma unroll
            for (int c = 0; c < C; ++c) sum += __builtin_bit_cast(f32x4_t, v[c]);
          }
          *(f32x4_t*)(sums + 4 * (r * nchk + q)) = sum;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < EPTM; ++s) {
          const int e = tid + kRecThreads * s;
          if (s < EPT && e < nel) {
            const int bl = e & (a.NB - 1), jj = e >> lgNB;
            const int q = bl * (a.NJ / 4) + (jj >> 2);
            float v = 0.f;
            for (int r = 0; r < tpc; ++r) v += sums[4 * (r * nchk + q) + (jj & 3)];
            dhc[s] = v;
          }
        }
        __syncthreads();
      }
    }
    const uint64_t* src = a.PX + ((int64_t)((t + 1) & 1) * nBG + bg) * a.nJG * HpNB;
    uint32_t off[C];
    uint32_t live = 0;
    uint64_t wv[C];
    if (VNCT > 0 && gather) {
      live = plan_dh_round<C>(off, 0, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
      issue_tagged<C>(wv, src, off);
    }
    if (VNCT > 0 && gather) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)(t + 2), a.err, dead);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float v = ((live >> c) & 1u) ? xval(wv[c]) : 0.f;
          if constexpr (EPTM == 1) {
            acc[0] += v;
          } else {
            const int slot = ((base / kRecThreads) + c) & (EPT - 1);
            acc[0] += slot == 0 ? v : 0.f;
            acc[1] += slot == 1 ? v : 0.f;
            acc[2] += slot == 2 ? v : 0.f;
            acc[3] += slot == 3 ? v : 0.f;
          }
        }
        base += kRecThreads * C;
        if (base >= gtotal) break;
        live = plan_dh_round<C>(off, base, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
        issue_tagged<C>(wv, src, off);
      }
      // sums[s][tid] holds this thread's part of element tid + 256*s (EPT > 1),
      // or of element tid % nel (TPE > 1)
#pragma unroll
      for (int s = 0; s < EPTM; ++s) sums[kRecThreads * s + tid] = acc[s];
      __syncthreads();
#pragma unroll
      for (int s = 0; s < EPTM; ++s) {
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
    wait_vmem();  // as in the forward: nothing of the last step is outstanding
    stamp(a.stamps, a.T, step, 1);

    // 2. gate deltas of this step
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
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
    if constexpr (VNCT > 0) {
      // NB == 4: pieces acc[i][column cc][batch row] over this lane's rows
      float acc[VNCT][4][4];
#pragma unroll
      for (int i = 0; i < VNCT; ++i)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[i][cc][0] = acc[i][cc][1] = acc[i][cc][2] = acc[i][cc][3] = 0.f;
#pragma unroll
      for (int r4 = 0; r4 < VRC / 4; ++r4) {
        f32x4_t dv[4];
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) dv[bl] = *(const f32x4_t*)(Dl + bl * strideD + (qp * VRC + 4 * r4) * 4);
#pragma unroll
        for (int i = 0; i < VNCT; ++i)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc)
#pragma unroll
            for (int bl = 0; bl < 4; ++bl)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) acc[i][cc][bl] = fmaf(wq[i][cc][4 * r4 + rr], dv[bl][rr], acc[i][cc][bl]);
      }
      const uint64_t tg = (uint64_t)(t + 1) << 32;
      const int qb1 = (qp >> 1) & 1, qb0 = qp & 1;
#pragma unroll
      for (int i = 0; i < VNCT; ++i) {
        // quad bit 1: keep columns 2*qb1 + {0,1}; bit 0: keep column qp
        float fin[4];
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
          float k2[2];
#pragma unroll
          for (int cl = 0; cl < 2; ++cl) {
            const float keep = qb1 ? acc[i][2 + cl][bl] : acc[i][cl][bl];
            const float send = qb1 ? acc[i][cl][bl] : acc[i][2 + cl][bl];
            k2[cl] = keep + quad_dpp<0x4E>(send);  // quad_perm [2,3,0,1]
          }
          const float keep = qb0 ? k2[1] : k2[0];
          const float send = qb0 ? k2[0] : k2[1];
          fin[bl] = keep + quad_dpp<0xB1>(send);  // quad_perm [1,0,3,2]
        }
        const int k = kRecThreads * i + 4 * qd + qp;
        if (k < a.H) {
          uint64_t* q = dst + (int64_t)k * 4;
          const uint64_t w0 = tg | __float_as_uint(fin[0]), w1 = tg | __float_as_uint(fin[1]);
          const uint64_t w2 = tg | __float_as_uint(fin[2]), w3 = tg | __float_as_uint(fin[3]);
          if (local) {
            // two 16-byte stores; each 8-byte word lands whole
            typedef __attribute__((__vector_size__(2 * sizeof(uint64_t)))) uint64_t u64x2_t;
            *(u64x2_t*)q = u64x2_t{w0, w1};
            *(u64x2_t*)(q + 2) = u64x2_t{w2, w3};
          } else {
            xstore_word(q, w0, false);
            xstore_word(q + 1, w1, false);
            xstore_word(q + 2, w2, false);
            xstore_word(q + 3, w3, false);
          }
        }
      }
    }
    if constexpr (VNCT == 0) for (int nt = 0; nt < NBT; ++nt) {
      u32x4_t breg[NKBR];
#pragma unroll
      for (int kb = 0; kb < NKBR; ++kb)
        breg[kb] = *(const u32x4_t*)(Dl + (16 * nt + fr) * strideD + kb * 64 + fq * 16);
      const int bl = 16 * nt + fr;
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKBR; ++kb) acc = Mfma<T>::mac(wreg[i * NKBR + kb], breg[kb], acc);
        if (bl < a.NB) {
          // 16 bytes: columns k0..k0+3 of row bl, packed
          const int k0 = 16 * (w + kWaves * i) + 4 * fq;
          float* q = a.PD + ((((int64_t)(t & 1) * nBG + bg) * a.nJG + jg) * a.NB + bl) * a.Hp + k0;
          if (local) {
            *(f32x4_t*)q = acc;
          } else {
            const uint64_t lo = (uint64_t)__float_as_uint(acc[0]) | ((uint64_t)__float_as_uint(acc[1]) << 32);
            const uint64_t hi = (uint64_t)__float_as_uint(acc[2]) | ((uint64_t)__float_as_uint(acc[3]) << 32);
            __hip_atomic_store((uint64_t*)q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store((uint64_t*)q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    if constexpr (VNCT == 0) {
      // publish: every partial of this work-group is stored, then the flag
      wait_vmem();
      __syncthreads();
      if (tid == 0) store_flag(a.PF + bg * a.nJG + jg, (uint32_t)(a.T - t), local);
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
  for (int s = 0; s < EPTM; ++s) {
    const int e = tid + kRecThreads * s;
    const int b = b0 + (e & (a.NB - 1)), uu = j0 + (e >> lgNB);
    if (s < EPT && e < nel && b < a.B && uu < a.H) {
      ((T*)a.dh0)[(int64_t)b * a.H + uu] = Elem<T>::from_f(dhc[s]);
      ((T*)a.dc0)[(int64_t)b * a.H + uu] = Elem<T>::from_f(dcc[s]);
    }
  }
}

// ---------------------------------------------------------------------------
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
  char* hd = (char*)HX;  // the packed ring and its flags share the tagged-word region
  FwdArgs a{P, W, h0, c0, y, hT, cT, Gs, Cs, HX, hd, (uint32_t*)(hd + p.off_hflags), (uint32_t)p.off_hflags, err,
            stamps, (int)p.T, (int)p.B, (int)p.H, (int)p.Z, p.NB, p.NJ,
            p.nJG, p.Hp, p.Bp, p.dtype ? (p.Hp / 2) : p.Hp, p.nBG, p.nxcd, p.xcd_local};
  if (fwd_vec_ok(p)) return launch_fwd_vec(p, a, s);
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
  char* pd = (char*)PX;
  BwdArgs a{W, c0, dy, dhT, dcT, Gs, Cs, dG, PX, (float*)pd, (uint32_t*)(pd + p.off_pflags), (uint32_t)p.off_pflags,
            DBP, dh0, dc0, err, stamps, (int)p.T, (int)p.B, (int)p.H, (int)p.Z,
            p.NB, p.NJ, p.nJG, p.Hp, p.Bp, p.nBG, p.nxcd, p.xcd_local};
  const int nkbr = 4 * p.NJ * p.esize / 64;
  if (p.dtype == 0 && p.NB == 4) {
    // VALU partial product: columns per thread x rows <= 128 resident floats
    // (spill-free instantiations only; other shapes take the MFMA form)
    const int vnct = p.Hp <= kRecThreads ? 1 : p.Hp / kRecThreads;
    const int C = p.words_per_thread <= 4 ? 4 : 16;
    if (p.NJ == 8 && C == 4) {
      if (vnct == 1) return coop_launch(bwd_rec_kernel<float, 1, 1, 4, 1, 32>, p.grid, p.lds_bwd, &a, s);
      if (vnct == 2) return coop_launch(bwd_rec_kernel<float, 1, 1, 4, 2, 32>, p.grid, p.lds_bwd, &a, s);
      if (vnct == 4) return coop_launch(bwd_rec_kernel<float, 1, 1, 4, 4, 32>, p.grid, p.lds_bwd, &a, s);
    }
    if (p.NJ == 8 && C == 16) {
      if (vnct == 1) return coop_launch(bwd_rec_kernel<float, 1, 1, 16, 1, 32>, p.grid, p.lds_bwd, &a, s);
      if (vnct == 2) return coop_launch(bwd_rec_kernel<float, 1, 1, 16, 2, 32>, p.grid, p.lds_bwd, &a, s);
      if (vnct == 4) return coop_launch(bwd_rec_kernel<float, 1, 1, 16, 4, 32>, p.grid, p.lds_bwd, &a, s);
    }
    if (p.NJ == 16 && vnct == 1) {
      if (C == 4) return coop_launch(bwd_rec_kernel<float, 1, 1, 4, 1, 64>, p.grid, p.lds_bwd, &a, s);
      return coop_launch(bwd_rec_kernel<float, 1, 1, 16, 1, 64>, p.grid, p.lds_bwd, &a, s);
    }
  }
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
