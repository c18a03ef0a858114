// recurrent.hip -- persistent forward recurrence, MFMA form (gfx950), and
// the dispatch of both recurrences.
//
// Forward ("SingleLayerLstmGrad" page, forward table): for t = 0..T-1
//   a_t = P_t + W_h h_{t-1}      (P_t = W_x x_t + b from the input projection)
//   i,f,o = sigmoid, g = tanh;   c_t = f c_{t-1} + i g;   h_t = o tanh(c_t)
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
// Exchange per step inside a batch group (flag exchange, see
// recurrent_common.hpp): every work-group writes h_t of its units into a
// two-slot ring of packed rows, waits for those stores, and sets its step
// flag; a reader waits for the flags of all work-groups of its group and
// then copies the group's rows of h_{t-1} into LDS with 16-byte loads.  No
// other grid-wide synchronisation is used.  In the XCD-local layout a batch
// group lives on one XCD and its ring stays in that XCD's L2.
//
// The backward recurrence is in recurrent_bwd.hip (MFMA form) and
// recurrent_vec.hip (VALU form for fp32 batch groups of 4 rows).
//
// Compile-time shapes (H is padded to Hp, a power of two): NKBW k-blocks of
// W_h per wave, NBT 16-row batch tiles, C ring chunks in flight per thread,
// NW waves (8-wave work-groups hold twice the W_h slice of 4-wave ones).
#include "recurrent_common.hpp"

namespace lstm {

// ---------------------------------------------------------------------------
template <typename T, int NBT, int NKBW, int C, int NW = kWaves>
__global__ void __launch_bounds__(64 * NW, 1) fwd_rec_kernel(FwdArgs a) {
  constexpr int NTH = 64 * NW;
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
  const int KS = NW / MT;                // waves splitting k per M-tile
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
  for (int idx = tid; idx < NBr * a.Hp; idx += NTH) {
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
      for (int idx = tid; idx < NBv * a.H; idx += NTH) {
        const int bl = idx / a.H, k = idx % a.H;
        const T v = a.h0 ? ((const T*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : T(0);
        *(T*)(Hl + bl * strideH + k * E) = v;
      }
    } else {
      const uint32_t slot0 = (uint32_t)(((t - 1) & 1) * a.Bp + b0) * (uint32_t)rowB;
      for (int q0 = 0; q0 < nchunk; q0 += NTH * C) {
        u32x4_t v[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int q = q0 + c * NTH + tid;
          const int bl = q / cpr, cc = q - bl * cpr;
          v[c] = q < nchunk ? load16_coherent(hd_rsrc, slot0 + (uint32_t)(bl * rowB + cc * 16)) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int q = q0 + c * NTH + tid;
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
template <typename T, int NBT, int C, int NW>
static hipError_t fwd_dispatch_c(const Plan& p, FwdArgs& a, hipStream_t s) {
  const int nt = 64 * NW;
  switch (p.fwd_nkbw) {
    case 1: return coop_launch(fwd_rec_kernel<T, NBT, 1, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
    case 2: return coop_launch(fwd_rec_kernel<T, NBT, 2, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
    case 4: return coop_launch(fwd_rec_kernel<T, NBT, 4, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
    case 8: return coop_launch(fwd_rec_kernel<T, NBT, 8, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
    case 16: return coop_launch(fwd_rec_kernel<T, NBT, 16, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
    case 32: return coop_launch(fwd_rec_kernel<T, NBT, 32, C, NW>, p.grid, p.lds_fwd, &a, s, nt);
  }
  return hipErrorInvalidValue;
}

// h chunks in flight per thread: as many as a thread reads per step (4 or
// 16), so that few load slots go unused; 8-wave work-groups (bf16 only)
// take 16
template <typename T, int NBT>
static hipError_t fwd_dispatch(const Plan& p, FwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2)
    if (p.waves == 8) return fwd_dispatch_c<T, NBT, 16, 8>(p, a, s);
  if (p.waves != kWaves) return hipErrorInvalidValue;
  if (p.words_per_thread <= 4) return fwd_dispatch_c<T, NBT, 4, kWaves>(p, a, s);
  return fwd_dispatch_c<T, NBT, 16, kWaves>(p, a, s);
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

hipError_t launch_bwd_recurrent(const Plan& p, const void* W, const void* c0, const void* dy, const void* dhT,
                                const void* dcT, const void* Gs, const float* Cs, void* dG, uint64_t* PX, float* DBP,
                                void* dh0, void* dc0, uint32_t* err, uint64_t* stamps, hipStream_t s) {
  char* gd = (char*)PX;  // the gate-delta ring and its flags share the tagged-word region
  BwdArgs a{W, c0, dy, dhT, dcT, Gs, Cs, dG, PX, gd, (uint32_t*)(gd + p.off_pflags), (uint32_t)p.off_pflags,
            DBP, dh0, dc0, err, stamps, (int)p.T, (int)p.B, (int)p.H, (int)p.Z,
            p.NB, p.NJ, p.nJG, p.Hp, p.Bp, p.nBG, p.nxcd, p.xcd_local};
  if (p.bwd_valu) return launch_bwd_vec(p, a, s);
  return launch_bwd_col(p, a, s);
}

}  // namespace lstm
