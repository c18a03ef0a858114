// recurrent_vec.hip -- forward and backward recurrences for fp32 storage
// with batch groups of 4 rows, the products on the vector ALUs (gfx950).
//
// Same step as the MFMA kernel ("SingleLayerLstmGrad" page, forward table:
// a_t = P_t + W_h h_{t-1}; i,f,o = sigmoid, g = tanh; c_t = f c_{t-1} + i g;
// h_t = o tanh(c_t)), but a 16x16 MFMA tile would leave 12 of its 16 batch
// columns empty for 4 rows.  Here:
//   lane c (0..31) of half-wave h of wave w owns local unit 2w + h (+ 8q for
//   q < U2 when NJ = 16): the four gate rows of the unit over the k-chunk c
//   of L = max(4, Hp/32) columns, kept in VGPRs for the whole launch;
//   h_{t-1} of the 4 rows sits in LDS as [row][chunk][L + 4] (the pad puts
//   neighbouring chunks on different banks);
//   each lane forms the 16 (gate, row) dot-product pieces of its chunk with
//   fp32 FMAs -- per FMA one LDS value feeds four gates, which keeps the
//   LDS reads (not the FMAs) from bounding the step;
//   the 32 chunks are summed by a reduce-scatter across the half-wave (xor
//   16 by v_permlane16_swap; xor 8, 4, 2, 1 by DPP), after which lane c holds the
//   full sum of gate 2*c[2] + c[1] for batch row 2*c[4] + c[3];
//   lane c = 8b (b < 4) gathers the four gates of batch row b by DPP and
//   does the cell update of that (unit, row) element.
// Both kernels exchange through tagged 8-byte words (value + step tag,
// relaxed agent-scope atomics, or plain stores in the XCD-local layout; see
// device_common.hpp), read with all of a thread's loads of a round in
// flight at once and only the words whose tag is not there yet polled again.
#include "recurrent_common.hpp"

namespace lstm {

// gfx9 DPP controls
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadBcast2 = 0xAA;  // quad_perm [2,2,2,2]
constexpr int kRowShl4 = 0x104, kRowShr4 = 0x114, kRowRor8 = 0x128;

// v from another lane by a DPP move; lanes outside bank_mask keep `old`.
template <int CTRL, int BANKS = 0xf>
__device__ __forceinline__ float dpp_f32(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, BANKS, false));
}
// v of lane l ^ 8 (inside a 16-lane row): a rotation of the row by 8.
__device__ __forceinline__ float xor8_f32(float v) { return dpp_f32<kRowRor8>(0.f, v); }
// v of lane l ^ 4: banks 1, 3 (lane bit 2 set) take from l - 4, banks 0, 2 from l + 4.
__device__ __forceinline__ float xor4_f32(float v) { return dpp_f32<kRowShl4, 0x5>(dpp_f32<kRowShr4, 0xA>(0.f, v), v); }
// One reduce-scatter level over lane bit 4 (within each 32-lane half):
// lanes with bit 4 clear get lo(l) + lo(l ^ 16), the others hi(l ^ 16) +
// hi(l).  v_permlane16_swap exchanges the odd 16-lane rows of its first
// operand with the even rows of its second: (lo, hi) becomes (lo.r0, hi.r0,
// lo.r2, hi.r2) and (lo.r1, hi.r1, lo.r3, hi.r3), whose sum is the level.
__device__ __forceinline__ float rs16_f32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

template <int L, int U2, int C>
__global__ void __launch_bounds__(kRecThreads, 1) fwd_vec_kernel(Launch<FwdArgs> LA) {
  extern __shared__ __attribute__((aligned(16))) float hl[];
  constexpr int CS = L + 4;    // chunk stride (floats)
  constexpr int RS = 32 * CS;  // row stride
  constexpr int LG_L = L == 4 ? 2 : L == 8 ? 3 : L == 16 ? 4 : 5;
  // the wave index is uniform (said so, it stays in scalar registers and the
  // branches on it are scalar branches: an s_waitcnt under a divergent branch
  // would run for every wave)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  FwdArgs a;
  const int wgi = slot_select(LA, a);
  int bg, jg;
  take_role(wgi, a.nBG, a.nJG, a.nxcd, a.local, a.misplace, bg, jg);
  claim_role(a.claims, bg * a.nJG + jg, a.err);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;  // NB == 4
  const int c = lane & 31, ulb = 2 * w + (lane >> 5);
  const int bit3 = (c >> 3) & 1, bit2 = (c >> 2) & 1, bit1 = (c >> 1) & 1;  // lane bits of the reduce-scatter
  const int64_t G4 = 4 * (int64_t)a.H;
  bool dead = false;

  // resident W_h: gates 0..3 of units j0 + ulb + 8q, columns of chunk c
  float wr[U2][4][L];
#pragma unroll
  for (int q = 0; q < U2; ++q) {
    const int ur = j0 + ulb + 8 * q;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float* wrow = (const float*)a.W + ((int64_t)gate_block(g, a.ijfo) * a.H + ur) * a.Z;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        const int k = c * L + i;
        wr[q][g][i] = (ur < a.H && k < a.H) ? wrow[k] : 0.f;
      }
    }
  }
  const int NBv = (a.B - b0) < 4 ? (a.B - b0) : 4;
  for (int idx = tid; idx < 4 * RS; idx += kRecThreads) hl[idx] = 0.f;

  // elementwise lanes: c = 8b -> batch row b
  const int bme_l = c >> 3;
  const bool ew = (c & 7) == 0 && bme_l < NBv;
  const int bme = b0 + bme_l;
  float cst[U2], hst[U2];  // state of this lane's elements
  f32x4_t pf[U2];
#pragma unroll
  for (int q = 0; q < U2; ++q) {
    const int u = j0 + ulb + 8 * q;
    cst[q] = !(ew && u < a.H) ? 0.f
             : a.c0f           ? a.c0f[(int64_t)bme * a.H + u]
             : a.c0            ? ((const float*)a.c0)[(int64_t)bme * a.H + u]
                               : 0.f;
    hst[q] = (ew && a.h0 && u < a.H) ? ((const float*)a.h0)[(int64_t)bme * a.H + u] : 0.f;
  }
  const int lenb = ew ? len_of(a.len, bme, a.T) : a.T;  // length of this lane's batch row
  auto load_p = [&](int tt) {
#pragma unroll
    for (int q = 0; q < U2; ++q) {
      const int u = j0 + ulb + 8 * q;
      pf[q] = (ew && tt < a.T && u < a.H)
                  ? *(const f32x4_t*)(a.P + ((int64_t)mem_t(tt, a.T, a.rev) * a.B + bme) * G4 + 4 * (int64_t)u)
                  : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_p(0);

  const int lgHW = 31 - __builtin_clz(a.HW);  // HW = Hp words per row
  const int total = NBv << lgHW;
  const uint32_t doff = (uint32_t)(tid % total);

  for (int t = 0; t < a.T; ++t) {
    stamp(a.stamps, a.T, t, 0);
    inject_failure(a.fail_step, t, wgi, a.err, dead);
    const uint64_t* src = a.HX + ((int64_t)((t - 1) & 1) * a.Bp + b0) * a.HW;
    uint32_t off[C];
    uint32_t live = 0;
    uint64_t wv[C];
    if (t > 0) {
      live = plan_h_round<C>(off, 0, tid, total, a.HW - 1, a.H, doff);
      issue_tagged<C>(wv, src, off);
    }
    __syncthreads();  // the previous step's readers of hl are done
    if (t == 0) {
      wait_vmem();
      for (int idx = tid; idx < NBv * a.H; idx += kRecThreads) {
        const int bl = idx / a.H, k = idx % a.H;
        hl[bl * RS + (k >> LG_L) * CS + (k & (L - 1))] = a.h0 ? ((const float*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : 0.f;
      }
    } else {
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)t, a.err, dead);
#pragma unroll
        for (int cc = 0; cc < C; ++cc) {
          if ((live >> cc) & 1u) {
            const int bl = off[cc] >> lgHW, k = off[cc] & (a.HW - 1);
            hl[bl * RS + (k >> LG_L) * CS + (k & (L - 1))] = xval(wv[cc]);
          }
        }
        base += kRecThreads * C;
        if (base >= total) break;
        live = plan_h_round<C>(off, base, tid, total, a.HW - 1, a.H, doff);
        issue_tagged<C>(wv, src, off);
      }
    }
    // Everything this wave issued before (last step's stores, the input
    // prefetch) has completed by now; saying so keeps the compiler from
    // waiting for stores before it reuses their registers below.
    wait_vmem();
    stamp(a.stamps, a.T, t, 1);
    __syncthreads();
    stamp(a.stamps, a.T, t, 2);

    // dot-product pieces of chunk c: acc[q][g][b]
    float acc[U2][4][4];
#pragma unroll
    for (int q = 0; q < U2; ++q)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[q][g][0] = acc[q][g][1] = acc[q][g][2] = acc[q][g][3] = 0.f;
    const float* hb = hl + c * CS;
#pragma unroll
    for (int i4 = 0; i4 < L / 4; ++i4) {
      f32x4_t hv[4];
#pragma unroll
      for (int bl = 0; bl < 4; ++bl) hv[bl] = *(const f32x4_t*)(hb + bl * RS + 4 * i4);
#pragma unroll
      for (int q = 0; q < U2; ++q)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int bl = 0; bl < 4; ++bl)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc[q][g][bl] = fmaf(wr[q][g][4 * i4 + kk], hv[bl][kk], acc[q][g][bl]);
    }
    stamp(a.stamps, a.T, t, 3);

    // reduce-scatter over the 32 chunk lanes; then gather the four gates
    f32x4_t z[U2];
#pragma unroll
    for (int q = 0; q < U2; ++q) {
      // bit 4: keep rows 2*bit4 + {0,1}
      float k8[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) k8[g][bb] = rs16_f32(acc[q][g][bb], acc[q][g][2 + bb]);
      // bit 3: keep row 2*bit4 + bit3
      float k4[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float keep = bit3 ? k8[g][1] : k8[g][0];
        const float send = bit3 ? k8[g][0] : k8[g][1];
        k4[g] = keep + xor8_f32(send);
      }
      // bit 2: keep gates 2*bit2 + {0,1}
      float k2[2];
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const float keep = bit2 ? k4[2 + gg] : k4[gg];
        const float send = bit2 ? k4[gg] : k4[2 + gg];
        k2[gg] = keep + xor4_f32(send);
      }
      // bit 1: keep gate 2*bit2 + bit1; bit 0: both lanes of the pair sum
      const float keep = bit1 ? k2[1] : k2[0];
      const float send = bit1 ? k2[0] : k2[1];
      float v = keep + dpp_f32<kQuadSwap2>(0.f, send);
      v += dpp_f32<kQuadSwap1>(0.f, v);
      // lane 8b + 2*bit2 + bit1 now holds gate 2*bit2 + bit1 of row b
      const float g1 = dpp_f32<kQuadBcast2>(0.f, v);  // from lane + 2
      z[q][0] = v;
      z[q][1] = g1;
      z[q][2] = dpp_f32<kRowShl4>(0.f, v);   // from lane + 4
      z[q][3] = dpp_f32<kRowShl4>(0.f, g1);  // from lane + 6
    }
    stamp(a.stamps, a.T, t, 4);

    if (ew) {
      uint64_t* dst = a.HX + (int64_t)(t & 1) * a.Bp * a.HW;
#pragma unroll
      for (int q = 0; q < U2; ++q) {
        const int u = j0 + ulb + 8 * q;
        if (u < a.H) {
          const f32x4_t zz = z[q] + pf[q];
          const float ig = sigmoidf(zz[0]), fg = sigmoidf(zz[1]), gg = tanh_f(zz[2]), og = sigmoidf(zz[3]);
          float cn = fg * cst[q] + ig * gg;
          float h = og * tanh_f(cn);
          if (mem_t(t, a.T, a.rev) >= lenb) {  // past the sequence's end: the state is held
            cn = cst[q];
            h = hst[q];
          }
          cst[q] = cn;
          hst[q] = h;
          xstore(dst + (int64_t)bme * a.HW + u, h, (uint32_t)(t + 1), local);
          const int64_t o = (int64_t)mem_t(t, a.T, a.rev) * a.B + bme;
          ((float*)a.y)[o * a.H + u] = h;
          *(f32x4_t*)((float*)a.Gs + o * G4 + 4 * (int64_t)u) = f32x4_t{ig, fg, gg, og};
          a.Cs[o * a.H + u] = cn;
          if (t == a.T - 1) {
            ((float*)a.hT)[(int64_t)bme * a.H + u] = h;
            ((float*)a.cT)[(int64_t)bme * a.H + u] = cn;
          }
        }
      }
    }
    load_p(t + 1);
    stamp(a.stamps, a.T, t, 5);
  }
}

// ---------------------------------------------------------------------------
// Backward ("SingleLayerLstmGrad" page, "反向传播算法" steps 1-6; the step is
// that of the MFMA kernel in recurrent_bwd.hip) with the partition by gate
// rows: work-group (bg, jg) forms, for its 4*NJ gate rows, the fp32 partial
// product W_h[rows]^T dG_t for all H columns and publishes it as tagged words
// [group][producer][column][row]; every work-group then sums, in a fixed
// order, the partials of its own units from all producers of the group.  At
// 4 batch rows the partials are few (nJG*4*NJ words per work-group and
// step), so this beats gathering the 4H gate deltas of every row.
//
// The partial product on the VALUs: lane quad qd = t/4 owns the W_h columns
// 256*i + 4*qd + {0..3} (i < VNCT), lane p = t%4 of the quad the row chunk
// [p*VR/4, (p+1)*VR/4) of the VR = 4*NJ rows of the work-group's units,
// kept in VGPRs.  Each lane forms the 16 (column, batch row) pieces of its
// chunk with fp32 FMAs -- one LDS value of dG feeds four columns -- and a
// reduce-scatter across the quad (DPP) leaves lane p with the four
// batch-row sums of column 256*i + 4*qd + p, stored as 32 contiguous bytes.
template <int VNCT, int VR, int C>
__global__ void __launch_bounds__(kRecThreads, 1) bwd_vec_kernel(Launch<BwdArgs> L) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  BwdArgs a;
  const int wgi = slot_select(L, a);
  int bg, jg;
  take_role(wgi, a.nBG, a.nJG, a.nxcd, a.local, a.misplace, bg, jg);
  claim_role(a.claims, bg * a.nJG + jg, a.err);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int nel = a.NB * a.NJ;               // (batch row, unit) elements: 32 or 64
  const int lgNB = 31 - __builtin_clz(a.NB), lgNel = 31 - __builtin_clz(nel);
  const int TPE = kRecThreads / nel;         // threads per element
  const int strideD = 4 * a.NJ * 4 + 16;
  char* Dl = smem;                                     // [4][strideD] gate deltas of the step
  float* sums = (float*)(smem + 4 * strideD);          // [kRecThreads] gather sums
  float* dba = sums + kRecThreads;                     // [nel][4] db: gate deltas summed over time
  for (int idx = tid; idx < 4 * nel; idx += kRecThreads) dba[idx] = 0.f;
  for (int idx = tid; idx < 4 * strideD / 4; idx += kRecThreads) ((uint32_t*)Dl)[idx] = 0u;
  const int64_t G4 = 4 * (int64_t)a.H;
  const int gtotal = a.nJG * nel;                      // exchange words read per step
  const int nBG = a.nBG;
  const int HpNB = a.Hp * a.NB;                        // words of one producer's block
  const uint32_t doff = (uint32_t)(tid % gtotal);      // target of unused load slots
  bool dead = false;

  constexpr int VRC = VR / 4;  // rows per quad lane
  float wq[VNCT][4][VRC];
  const int qd = tid >> 2, qp = tid & 3;
#pragma unroll
  for (int i = 0; i < VNCT; ++i)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int k = kRecThreads * i + 4 * qd + cc;
#pragma unroll
      for (int rr = 0; rr < VRC; ++rr) {
        const int r = qp * VRC + rr, ur = j0 + (r >> 2), g = r & 3;
        wq[i][cc][rr] =
            (k < a.H && ur < a.H) ? ((const float*)a.W)[((int64_t)gate_block(g, a.ijfo) * a.H + ur) * a.Z + k] : 0.f;
      }
    }

  // elementwise ownership: thread tid < nel owns element e = tid (batch row
  // fastest); every thread takes part in the gather
  const int e = tid;
  const int bl0 = e & (a.NB - 1), jj0 = e >> lgNB;
  const int bown = b0 + bl0, uown = j0 + jj0;
  const bool own = e < nel && bown < a.B && uown < a.H;
  const int64_t BH = (int64_t)a.B * a.H;
  float dcc = !own ? 0.f : a.carry_in ? a.carry[BH + (int64_t)bown * a.H + uown]
                   : a.dcT ? ((const float*)a.dcT)[(int64_t)bown * a.H + uown] : 0.f;
  float dhc = !own ? 0.f : a.carry_in ? a.carry[(int64_t)bown * a.H + uown]
                   : a.dhT ? ((const float*)a.dhT)[(int64_t)bown * a.H + uown] : 0.f;
  // dh of a step past the sequence's end reaches the held state unchanged
  float pass = 0.f;
  const int lenb = own ? len_of(a.len, bown, a.T) : a.T;

  // elementwise operands of a step (activated gates, c_t, c_{t-1}, dy_t),
  // prefetched one step ahead
  float pg[4], pc, pcp, pdy;
  const int64_t g_off = (int64_t)bown * G4 + 4 * (int64_t)uown, c_off = (int64_t)bown * a.H + uown;
  const int64_t stepG = (int64_t)a.B * G4, stepC = (int64_t)a.B * a.H;
  auto load_ops = [&](int tt) {
    pg[0] = pg[1] = pg[2] = pg[3] = 0.f;
    pc = pcp = pdy = 0.f;
    if (tt >= 0 && own) {
      const int tm = mem_t(tt, a.T, a.rev);
      const int64_t oG = (int64_t)tm * stepG, oC = (int64_t)tm * stepC;
      const f32x4_t gv = *(const f32x4_t*)((const float*)a.Gs + oG + g_off);
      pg[0] = gv[0]; pg[1] = gv[1]; pg[2] = gv[2]; pg[3] = gv[3];
      pc = a.Cs[oC + c_off];
      pcp = tt > 0 ? a.Cs[(int64_t)mem_t(tt - 1, a.T, a.rev) * stepC + c_off]
                   : a.cprevf ? a.cprevf[c_off] : (a.c0 ? ((const float*)a.c0)[c_off] : 0.f);
      pdy = ((const float*)a.dy)[oC + c_off];
    }
  };
  load_ops(a.T - 1);

  for (int t = a.T - 1; t >= -1; --t) {
    const int step = a.T - 1 - (t < 0 ? 0 : t);
    if (t >= 0) stamp(a.stamps, a.T, step, 0);
    if (t >= 0) inject_failure(a.fail_step, step, wgi, a.err, dead);
    // 1. gather dh_carry: sum over work-groups of the partials produced at
    //    step t+1.  Word idx = jg' * nel + e (e = jj * NB + bl): a thread
    //    always meets the same element, in increasing jg' order, and the TPE
    //    threads sharing an element are then added in a fixed order.
    const bool gather = t < a.T - 1;
    if (!gather) wait_vmem();
    const uint64_t* src = a.PX + ((int64_t)((t + 1) & 1) * nBG + bg) * a.nJG * HpNB;
    if (gather) {
      uint32_t off[C];
      uint64_t wv[C];
      uint32_t live = plan_dh_round<C>(off, 0, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
      issue_tagged<C>(wv, src, off);
      float acc = 0.f;
      for (int base = 0;;) {
        complete_tagged<C>(wv, src, off, live, (uint32_t)(t + 2), a.err, dead);
#pragma unroll
        for (int c = 0; c < C; ++c) acc += ((live >> c) & 1u) ? xval(wv[c]) : 0.f;
        base += kRecThreads * C;
        if (base >= gtotal) break;
        live = plan_dh_round<C>(off, base, tid, gtotal, nel, lgNel, a.NB, lgNB, j0, b0, a.B, a.H, HpNB, doff);
        issue_tagged<C>(wv, src, off);
      }
      // sums[tid] holds this thread's part of element tid % nel
      sums[tid] = acc;
      __syncthreads();
      if (e < nel) {
        float v = 0.f;
        for (int q = 0; q < TPE; ++q) v += sums[tid + q * nel];
        dhc = v + pass;
      }
      __syncthreads();
    }
    if (t < 0) break;
    wait_vmem();  // nothing of the last step is outstanding
    stamp(a.stamps, a.T, step, 1);

    // 2. gate deltas of this step
    if (e < nel) {
      f32x4_t dq = {0.f, 0.f, 0.f, 0.f};
      if (own) {
        const int64_t o = (int64_t)mem_t(t, a.T, a.rev) * a.B + bown;
        const float gi = pg[0], gf = pg[1], gg = pg[2], go = pg[3];
        const float tc = tanh_f(pc);
        const float dh = pdy + dhc;
        const bool live = mem_t(t, a.T, a.rev) < lenb;
        const float m = live ? 1.f : 0.f;
        const float dc = dh * go * (1.f - tc * tc) + dcc;
        const float d_o = m * (dh * tc * go * (1.f - go));
        const float d_g = m * (dc * gi * (1.f - gg * gg));
        const float d_i = m * (dc * gg * gi * (1.f - gi));
        const float d_f = m * (dc * pcp * gf * (1.f - gf));
        dcc = live ? dc * gf : dcc;
        pass = live ? 0.f : dh;
        dq = f32x4_t{d_i, d_f, d_g, d_o};
        *(f32x4_t*)(dba + 4 * e) += dq;
        *(f32x4_t*)((float*)a.dG + o * G4 + 4 * (int64_t)uown) = dq;
      }
      *(f32x4_t*)(Dl + bl0 * strideD + jj0 * 16) = dq;
    }
    __syncthreads();
    stamp(a.stamps, a.T, step, 2);

    // 3. partial[k][b] = sum_{r in my rows} W_h[r][k] dG[b][r], all k < H:
    //    pieces acc[i][column cc][batch row] over this lane's rows
    uint64_t* dst = a.PX + (((int64_t)(t & 1) * nBG + bg) * a.nJG + jg) * HpNB;
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
          k2[cl] = keep + quad_dpp<kQuadSwap2>(send);
        }
        const float keep = qb0 ? k2[1] : k2[0];
        const float send = qb0 ? k2[0] : k2[1];
        fin[bl] = keep + quad_dpp<kQuadSwap1>(send);
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
  if (own && a.carry_out) {
    a.carry[c_off] = dhc;
    a.carry[BH + c_off] = dcc;
  } else if (own) {
    ((float*)a.dh0)[c_off] = dhc;
    ((float*)a.dc0)[c_off] = dcc;
  }
}

// Dispatch: L = max(4, Hp/32) columns per chunk, U2 = NJ/8 units per
// half-wave; the resident slice 4*U2*L floats per lane is kept at most 64
// (larger slices spill with the fully unrolled product).
static int vec_chunk(const Plan& p) { return p.Hp / 32 < 4 ? 4 : p.Hp / 32; }

bool fwd_vec_ok(const Plan& p) {
  if (p.dtype != 0 || p.NB != 4 || p.waves != kWaves) return false;
  const int L = vec_chunk(p), u2 = p.NJ / 8;
  return L <= 16 && (u2 == 1 || u2 == 2) && 4 * u2 * L <= 64;
}

template <int U2, int C>
static hipError_t fwd_vec_l(const Plan& p, Launch<FwdArgs>& a, hipStream_t s) {
  const int L = vec_chunk(p);
  const size_t lds = (size_t)4 * 32 * (L + 4) * sizeof(float);
  switch (L) {
    case 4: return coop_launch(fwd_vec_kernel<4, U2, C>, launch_grid(p, a), lds, &a, s);
    case 8: return coop_launch(fwd_vec_kernel<8, U2, C>, launch_grid(p, a), lds, &a, s);
    case 16:
      if constexpr (U2 == 1) return coop_launch(fwd_vec_kernel<16, U2, C>, launch_grid(p, a), lds, &a, s);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_vec(const Plan& p, Launch<FwdArgs>& a, hipStream_t s) {
  // exchange words a thread reads per step: 4*Hp/256 (at most 16)
  const bool wide = p.words_per_thread > 4;
  if (p.NJ == 8) return wide ? fwd_vec_l<1, 16>(p, a, s) : fwd_vec_l<1, 4>(p, a, s);
  return wide ? fwd_vec_l<2, 16>(p, a, s) : fwd_vec_l<2, 4>(p, a, s);
}

// Backward: VNCT = Hp/256 column groups per thread (at least 1), VR = 4*NJ
// rows; the make_plan conditions (NJ = 8 with VNCT <= 4, or NJ = 16 with
// VNCT = 1) keep the resident VNCT*4*VR/4 floats per lane at most 128.
hipError_t launch_bwd_vec(const Plan& p, Launch<BwdArgs>& a, hipStream_t s) {
  const int vnct = p.Hp <= kRecThreads ? 1 : p.Hp / kRecThreads;
  const bool wide = p.words_per_thread > 4;
  if (p.NJ == 8) {
    if (vnct == 1) return coop_launch(wide ? bwd_vec_kernel<1, 32, 16> : bwd_vec_kernel<1, 32, 4>, launch_grid(p, a), p.lds_bwd, &a, s);
    if (vnct == 2) return coop_launch(wide ? bwd_vec_kernel<2, 32, 16> : bwd_vec_kernel<2, 32, 4>, launch_grid(p, a), p.lds_bwd, &a, s);
    if (vnct == 4) return coop_launch(wide ? bwd_vec_kernel<4, 32, 16> : bwd_vec_kernel<4, 32, 4>, launch_grid(p, a), p.lds_bwd, &a, s);
  }
  if (p.NJ == 16 && vnct == 1)
    return coop_launch(wide ? bwd_vec_kernel<1, 64, 16> : bwd_vec_kernel<1, 64, 4>, launch_grid(p, a), p.lds_bwd, &a, s);
  return hipErrorInvalidValue;
}

}  // namespace lstm
