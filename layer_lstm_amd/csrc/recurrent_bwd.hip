// recurrent_bwd.hip -- persistent backward recurrence, MFMA form (gfx950).
//
// Step ("SingleLayerLstmGrad" page, "反向传播算法" steps 1-6), t = T-1..0:
//   dh = dy_t + dh_carry;  dc = dh o (1 - tanh^2 c_t) + dc_carry
//   do = dh tanh(c_t) o(1-o); dg = dc i (1-g^2); di = dc g i(1-i);
//   df = dc c_{t-1} f(1-f);  dc_carry = dc f;  dh_carry = W_h^T dG_t
// with the carries starting from dhT/dcT; dh0/dc0 are the carries left
// after t = 0.  The operands of the elementwise chain (activated gates, c_t,
// c_{t-1}) come from the forward's record.
//
// Partition by columns of W_h: work-group (bg, jg) owns batch rows
// [bg*NB, +NB) and hidden units [jg*NJ, +NJ) and keeps, as MFMA A
// fragments, W_h^T restricted to its units: the NJ columns of W_h over all
// 4H gate rows -- as many values as the forward's slice of 4*NJ rows.  Per
// step it
//   1. waits until every work-group of its batch group has published dG_{t+1}
//      (one step flag per producer) and forms dh_carry[b][u] for its units
//      completely: D[u][b] = sum_r W_h[r][u] dG_{t+1}[b][r] over r < 4H, the
//      waves splitting r and streaming their slice of dG_{t+1} from the
//      exchange ring straight into MFMA B fragments (two chunks of loads in
//      flight), then summing their partial tiles through LDS in a fixed
//      order;
//   2. runs the elementwise chain for its (row, unit) elements, writes dG_t
//      (for the dW / dx products) and publishes it into the ring slot t&1,
//      then its step flag.
// Nothing is summed across work-groups, so every work-group reads only
// dG values (NB * 4H per step, shared by the nJG readers of a batch group
// in L2) and writes only its own 4*NJ columns of them.
//
// Ring layout, in MFMA fragment order: a slot holds, for each batch group
// and each of its 16-row batch tiles, the 4Hp gate deltas (interleaved gates,
// gate row r = 4u + g) of the tile's rows as Hp*E/16 chunks of 1 KB; chunk kc
// holds the 64 bytes of gate rows [kc*64/E, +64/E) of each row, lane l = 16q
// + f of the B fragment (tile row f, bytes [16q, +16) of the chunk's rows) at
// bytes [16l, +16).  A wave's fragment load is one contiguous kilobyte.
// Gate rows past 4H are never written and stay zero (the ring is cleared
// before the forward and after every backward); B fragments of tile rows
// past NB are read out of the buffer's range, which returns zeros.
#include "recurrent_common.hpp"

namespace lstm {

// NBT 16-row batch tiles, MT 16-unit tiles, NKB k-blocks (16 bytes per lane
// each) of the 4Hp gate rows per wave, NW waves.  EPTM elements (row, unit)
// per thread at most.  DEF selects where the step's other memory traffic
// goes (see below).
template <typename T, int NBT, int MT, int NKB, int NW, bool DEF>
__global__ void __launch_bounds__(64 * NW, 1) bwd_col_kernel(Launch<BwdArgs> L) {
  constexpr int NTH = 64 * NW;
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  constexpr int EPTM = 1024 / NTH;                    // NB * NJ <= 1024
  // k-blocks per load chunk: two chunks of B fragments (2*CK*NBT*4 VGPRs) are
  // in flight next to the resident W_h^T slice (MT*NKB*4 VGPRs)
  constexpr int CKM = (MT * NKB >= 32 ? 4 : 8) / NBT > 0 ? (MT * NKB >= 32 ? 4 : 8) / NBT : 1;
  constexpr int CK = NKB < CKM ? NKB : CKM;
  constexpr int NCH = NKB / CK;
  constexpr int NJS = 16 * MT + 4;                    // LDS row of a wave's partial tile (floats)
  static_assert(NKB % CK == 0, "chunks divide the k-blocks");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the wave index is uniform (said so, it stays in scalar registers and the
  // branches on it are scalar branches: an s_waitcnt under a divergent branch
  // would run for every wave)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  BwdArgs a;
  const int wgi = slot_select(L, a);
  int bg, jg;
  take_role(wgi, a.nBG, a.nJG, a.nxcd, a.local, a.misplace, bg, jg);
  claim_role(a.claims, bg * a.nJG + jg, a.err);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int lgNJ = 31 - __builtin_clz(a.NJ);
  const int nel = a.NB * a.NJ;
  constexpr int NBr = 16 * NBT;
  float* red = (float*)smem;                          // [NW][NBr][NJS] per-wave partial dh
  float* dba = red + NW * NBr * NJS;                  // [nel][4] db: gate deltas summed over time
  const int64_t G4 = 4 * (int64_t)a.H;
  constexpr uint32_t kTileB = (uint32_t)NW * NKB * 1024; // bytes of one 16-row tile of the ring
  const __amdgpu_buffer_rsrc_t gd_rsrc = make_rsrc(a.GD, a.gd_bytes);
  bool dead = false;

  // --- resident A fragments: W_h^T[unit j0 + 16*mt + fr][gate row r], r =
  // (w*NKB + i)*KB + fq*16/E + e (interleaved: unit r/4, gate r%4).  W_h is
  // row-major, so the fragments are gathered through LDS: in each pass the
  // work-group reads PB k-blocks of every wave's rows (the units' columns of
  // a row are contiguous), stores them transposed as [unit][row], and every
  // lane then takes each of its fragments with one 16-byte LDS read.
  u32x4_t wreg[MT][NKB];
  {
    constexpr int PB0 = 65536 / (16 * MT * NW * KB * E);
    constexpr int PB = NKB < PB0 ? NKB : PB0;           // k-blocks per wave per pass
    constexpr int RS = NW * PB * KB + 16 / E;           // staged row (elements), padded
    constexpr int LPT = 16 * MT * PB * KB / 64;         // elements each thread loads per pass
    constexpr int RSTEP = NTH / (16 * MT);              // staged rows between a thread's loads
    static_assert((size_t)16 * MT * RS * E <= kColStageLds, "staging fits");
    T* stage = (T*)smem;
    const int ul = tid % (16 * MT), u = j0 + ul;        // the one unit this thread loads
    const bool uok = ul < a.NJ && u < a.H;
#pragma unroll
    for (int p = 0; p < NKB / PB; ++p) {
      T v[LPT];
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int rl = tid / (16 * MT) + j * RSTEP;     // staged row
        const int r = ((rl / (PB * KB)) * NKB + p * PB) * KB + rl % (PB * KB);
        const int ur = r >> 2, g = r & 3;
        const bool ok = uok && ur < a.H;
        v[j] = ((const T*)a.W)[ok ? ((int64_t)gate_block(g, a.ijfo) * a.H + ur) * a.Z + u : 0];
        v[j] = ok ? v[j] : T(0);
      }
      __syncthreads();  // the previous pass's fragment reads are done
#pragma unroll
      for (int j = 0; j < LPT; ++j) stage[ul * RS + tid / (16 * MT) + j * RSTEP] = v[j];
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ii = 0; ii < PB; ++ii)
          wreg[mt][p * PB + ii] = *(const u32x4_t*)(stage + (16 * mt + fr) * RS + (w * PB + ii) * KB + fq * (16 / E));
    }
    __syncthreads();  // the staging area is reused below
  }
  // ring byte offset (slot 0) of this lane's B fragments: tile nt of the
  // batch group, chunk w*NKB; tile rows past NB point out of the buffer (zeros)
  uint32_t boff[NBT];
#pragma unroll
  for (int nt = 0; nt < NBT; ++nt)
    boff[nt] = 16 * nt + fr < a.NB ? (uint32_t)(bg * NBT + nt) * kTileB + (uint32_t)(w * NKB * 1024 + lane * 16)
                                   : 0xC0000000u;
  const uint32_t slotB = (uint32_t)a.nBG * NBT * kTileB;

  // --- elementwise ownership: element e = tid + NTH*s (s < EPTM), unit fastest
  // (b, u) of element e and its offset in [B][H] tensors; in [B][4H] tensors
  // it is 4x that
  auto elem_b = [&](int s) { return b0 + ((tid + NTH * s) >> lgNJ); };
  auto elem_u = [&](int s) { return j0 + ((tid + NTH * s) & (a.NJ - 1)); };
  auto c_off = [&](int s) { return (uint32_t)elem_b(s) * (uint32_t)a.H + (uint32_t)elem_u(s); };
  float dcc[EPTM], dhc[EPTM];
  // pass: dh of a step past the sequence's end, which reaches the held
  // state unchanged (added to the next carry); lens: the row's length
  float pass[EPTM];
  int lens[EPTM];
  bool own[EPTM];
#pragma unroll
  for (int s = 0; s < EPTM; ++s) {
    const int e = tid + NTH * s;
    own[s] = e < nel && elem_b(s) < a.B && elem_u(s) < a.H;
    pass[s] = 0.f;
    lens[s] = own[s] ? len_of(a.len, elem_b(s), a.T) : a.T;
    const int64_t BH = (int64_t)a.B * a.H;
    dcc[s] = !own[s] ? 0.f : a.carry_in ? a.carry[BH + c_off(s)] : a.dcT ? ldf<T>(a.dcT, c_off(s)) : 0.f;
    dhc[s] = !own[s] ? 0.f : a.carry_in ? a.carry[c_off(s)] : a.dhT ? ldf<T>(a.dhT, c_off(s)) : 0.f;
    if (e < nel) *(f32x4_t*)(dba + 4 * e) = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Memory traffic off the exchange path: the operands of a step's
  // elementwise chain (activated gates, c_t, c_{t-1}, dy_t) are fetched one
  // step ahead, and the record of a step (dG rows for the dW / dx products)
  // is written.  A wave's vector-memory operations complete in issue order,
  // so this traffic delays whichever wait on the exchange comes next after
  // it is issued; where it goes depends on the exchange:
  //   DEF (XCD-local groups: the ring sits in L2 and the flag wait is short):
  //     issued as soon as the product's ring reads are consumed (into a
  //     second set of registers, the record one step late), it drains
  //     during the reduction and the gate deltas.  (Direct-to-LDS loads of
  //     the same operands held the waves up at the reduction's barrier,
  //     about a fifth of the step at 32-row groups.);
  //   !DEF (groups across XCDs: every flag and ring read goes through memory
  //     and the flag wait is long): the record is written with the ring and
  //     the operands are loaded into registers right after the flag, while
  //     the other work-groups' flags are on their way.
  constexpr int GSB = 4 * E;                                 // bytes of one element's gates
  const int64_t stepC = (int64_t)a.B * a.H;                  // elements of one step in [B][H]
  T pdy[EPTM], pdyn[EPTM];  // dy_t (in use), dy of the next step: raw, converted at use (a conversion at
                            // load time would make the load's issue wait for its data)
  uint32_t dqw[EPTM][GSB / 4];                               // this step's gate deltas, packed
  uint32_t rgw[EPTM][GSB / 4], ngw[EPTM][GSB / 4];           // gates of this step and of the next, raw
  float rc[EPTM], rcp[EPTM], nc[EPTM], ncp[EPTM];            // c_t, c_{t-1} of this step and of the next
  // operands of step tt >= 0 into registers (raw: no conversion at load
  // time, which would make the issue wait for the data): !DEF into the set
  // of this step, DEF into the set of the next
  auto load_ops = [&](int tt, uint32_t (&gw)[EPTM][GSB / 4], float (&cc)[EPTM], float (&cp)[EPTM], T (&dyv)[EPTM]) {
    if (tt < 0) return;
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
      if (!own[s]) continue;
      const int64_t o = (int64_t)mem_t(tt, a.T, a.rev) * stepC + c_off(s);
      if constexpr (E == 4) {
        const u32x4_t g = *(const u32x4_t*)((const T*)a.Gs + 4 * o);
        gw[s][0] = g[0]; gw[s][1] = g[1]; gw[s][2] = g[2]; gw[s][3] = g[3];
      } else {
        const uint64_t g = *(const uint64_t*)((const T*)a.Gs + 4 * o);
        gw[s][0] = (uint32_t)g; gw[s][1] = (uint32_t)(g >> 32);
      }
      cc[s] = a.Cs[o];
      cp[s] = tt > 0 ? a.Cs[(int64_t)mem_t(tt - 1, a.T, a.rev) * stepC + c_off(s)] : 0.f;
      dyv[s] = ((const T*)a.dy)[o];
    }
  };
  auto load_regs = [&](int tt) { load_ops(tt, rgw, rc, rcp, pdy); };
  auto issue_ops = [&](int tt) { load_ops(tt, ngw, nc, ncp, pdyn); };
  auto take_next = [&]() {
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
#pragma unroll
      for (int k = 0; k < GSB / 4; ++k) rgw[s][k] = ngw[s][k];
      rc[s] = nc[s];
      rcp[s] = ncp[s];
      pdy[s] = pdyn[s];
    }
  };
  auto store_record = [&](int tt) {
    // gate deltas of step tt into the dG record
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
      if (!own[s]) continue;
      T* dst = (T*)a.dG + 4 * ((int64_t)mem_t(tt, a.T, a.rev) * stepC + c_off(s));
      if constexpr (E == 4)
        *(u32x4_t*)dst = u32x4_t{dqw[s][0], dqw[s][1], dqw[s][2], dqw[s][3]};
      else
        *(uint64_t*)dst = (uint64_t)dqw[s][0] | ((uint64_t)dqw[s][1] << 32);
    }
  };
  load_regs(a.T - 1);

  for (int t = a.T - 1; t >= -1; --t) {
    const int step = a.T - 1 - (t < 0 ? 0 : t);
    if (t >= 0) stamp(a.stamps, a.T, step, 0);
    if (t >= 0) inject_failure(a.fail_step, step, wgi, a.err, dead);
    if (t < a.T - 1) {
      // 1. dh_carry = W_h^T dG_{t+1} for this group's units, complete
      if (tid < a.nJG) wait_flag(a.GF + bg * a.nJG + tid, (uint32_t)(a.T - t - 1), a.err, dead);
      __syncthreads();
      if (t >= 0) stamp(a.stamps, a.T, step, 1);
      const uint32_t sb = (uint32_t)((t + 1) & 1) * slotB;
      f32x4_t acc[MT][NBT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NBT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u32x4_t bb[2][CK][NBT];
      auto issue = [&](int ch, int buf) {
#pragma unroll
        for (int i = 0; i < CK; ++i)
#pragma unroll
          for (int nt = 0; nt < NBT; ++nt)
            bb[buf][i][nt] = load16_coherent(gd_rsrc, sb + boff[nt] + (uint32_t)((ch * CK + i) * 1024));
      };
      // scheduling barriers pin each chunk's loads ahead of the products of
      // the chunk before (the scheduler would otherwise trade loads in
      // flight for registers).  The deferred operations wait until every
      // ring read is consumed: with other kinds of operations outstanding
      // (stores, direct-to-LDS loads), the compiler can only wait for all.
      issue(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        if (ch + 1 < NCH) issue(ch + 1, (ch + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CK; ++i)
#pragma unroll
          for (int nt = 0; nt < NBT; ++nt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt][nt] = Mfma<T>::mac(wreg[mt][ch * CK + i], bb[ch & 1][i][nt], acc[mt][nt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DEF) {
        store_record(t + 1);
        issue_ops(t - 1);
      }
      // lane holds D[unit 16*mt + 4*fq + q][row 16*nt + fr], q < 4
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NBT; ++nt)
          *(f32x4_t*)(red + (w * NBr + 16 * nt + fr) * NJS + 16 * mt + 4 * fq) = acc[mt][nt];
      if (t >= 0) stamp(a.stamps, a.T, step, 2);
      // LDS writes done, then the barrier (not __syncthreads: that would also
      // wait for the deferred memory operations)
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int s = 0; s < EPTM; ++s) {
        const int e = tid + NTH * s;
        if (e < nel) {
          const int bl = e >> lgNJ, jj = e & (a.NJ - 1);
          float v = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) v += red[(w2 * NBr + bl) * NJS + jj];
          dhc[s] = v + pass[s];
        }
      }
    } else {
      if constexpr (DEF) issue_ops(t - 1);
      stamp(a.stamps, a.T, step, 1);
      stamp(a.stamps, a.T, step, 2);
    }
    if (t < 0) break;
    stamp(a.stamps, a.T, step, 3);

    // 2. gate deltas of this step; dG_t to the ring (the record follows next
    //    step)
    char* ring = (char*)a.GD + (t & 1) * slotB;
#pragma unroll
    for (int s = 0; s < EPTM; ++s) {
      uint32_t gw[GSB / 4];
#pragma unroll
      for (int k = 0; k < GSB / 4; ++k) gw[k] = rgw[s][k];
      float c = rc[s], cprev = rcp[s];
      float gi, gf, gg, go;
      if constexpr (E == 4) {
        gi = __uint_as_float(gw[0]); gf = __uint_as_float(gw[1]); gg = __uint_as_float(gw[2]); go = __uint_as_float(gw[3]);
      } else {
        gi = f_of_bits16<T>(gw[0]); gf = f_of_bits16<T>(gw[0] >> 16);
        gg = f_of_bits16<T>(gw[1]); go = f_of_bits16<T>(gw[1] >> 16);
      }
      if (t == 0)
        cprev = !own[s] ? 0.f : a.cprevf ? a.cprevf[c_off(s)] : a.c0 ? ldf<T>(a.c0, c_off(s)) : 0.f;
      const float tc = tanh_f(c);
      const float dh = Elem<T>::to_f(pdy[s]) + dhc[s];
      // past the sequence's end the step held the state: no gate deltas,
      // the cell carry unchanged, dh passed on to the next carry
      const bool live = mem_t(t, a.T, a.rev) < lens[s];
      const float m = live ? 1.f : 0.f;
      const float dc = dh * go * (1.f - tc * tc) + dcc[s];
      const float d_o = m * (dh * tc * go * (1.f - go));
      const float d_g = m * (dc * gi * (1.f - gg * gg));
      const float d_i = m * (dc * gg * gi * (1.f - gi));
      const float d_f = m * (dc * cprev * gf * (1.f - gf));
      pass[s] = live ? 0.f : dh;
      T dq[4] = {Elem<T>::from_f(d_i), Elem<T>::from_f(d_f), Elem<T>::from_f(d_g), Elem<T>::from_f(d_o)};
      if constexpr (E == 4) {
        const u32x4_t v = __builtin_bit_cast(u32x4_t, dq);
        dqw[s][0] = v[0]; dqw[s][1] = v[1]; dqw[s][2] = v[2]; dqw[s][3] = v[3];
      } else {
        const uint64_t v = __builtin_bit_cast(uint64_t, dq);
        dqw[s][0] = (uint32_t)v; dqw[s][1] = (uint32_t)(v >> 32);
      }
      if (own[s]) {
        if constexpr (!DEF) {
          T* dst = (T*)a.dG + 4 * ((int64_t)mem_t(t, a.T, a.rev) * stepC + c_off(s));
          if constexpr (E == 4)
            *(u32x4_t*)dst = __builtin_bit_cast(u32x4_t, dq);
          else
            *(uint64_t*)dst = __builtin_bit_cast(uint64_t, dq);
        }
        dcc[s] = live ? dc * gf : dcc[s];
        *(f32x4_t*)(dba + 4 * (tid + NTH * s)) += f32x4_t{d_i, d_f, d_g, d_o};
        // gate rows 4u..4u+3 of row bl: chunk kc, bytes [o, o + 4E) of it
        const uint32_t bl = (uint32_t)(elem_b(s) - b0), ob = 4u * E * (uint32_t)elem_u(s);
        const uint32_t kc = ob >> 6, o = ob & 63;
        T* rp = (T*)(ring + (uint32_t)(bg * NBT + (bl >> 4)) * kTileB + kc * 1024 +
                     ((o >> 4) * 16 + (bl & 15)) * 16 + (o & 15));
        if constexpr (E == 4) {
          if (local) {
            *(u32x4_t*)rp = __builtin_bit_cast(u32x4_t, dq);
          } else {
            const uint64_t lo = (uint64_t)dqw[s][0] | ((uint64_t)dqw[s][1] << 32);
            const uint64_t hi = (uint64_t)dqw[s][2] | ((uint64_t)dqw[s][3] << 32);
            __hip_atomic_store((uint64_t*)rp, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store((uint64_t*)rp + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          const uint64_t v = __builtin_bit_cast(uint64_t, dq);
          if (local)
            *(uint64_t*)rp = v;
          else
            __hip_atomic_store((uint64_t*)rp, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    // publish: every gate delta of this work-group is in the ring, then the flag
    wait_vmem();
    __syncthreads();
    if (tid == 0) store_flag(a.GF + bg * a.nJG + jg, (uint32_t)(a.T - t), local);
    if constexpr (DEF) {
      take_next();
    } else {
      // loaded to completion here, while the flags of this step travel: in
      // flight, the loads would hold up the next step's flag polls and ring
      // reads, which complete only after every earlier load of their wave
      load_regs(t - 1);
      wait_vmem();
    }
    stamp(a.stamps, a.T, step, 4);
    stamp(a.stamps, a.T, step, 5);
  }

  // db partial of this work-group: for each (unit, gate), the sum over its
  // batch rows (in row order) of the per-element sums over time
  if (a.DBP) {
    __syncthreads();
    for (int r = tid; r < 4 * a.NJ; r += NTH) {
      const int jj = r >> 2, g = r & 3;
      float v = 0.f;
      for (int bl = 0; bl < a.NB; ++bl) v += dba[4 * ((bl << lgNJ) + jj) + g];
      if (j0 + jj < a.H) a.DBP[(int64_t)bg * G4 + 4 * (j0 + jj) + g] = v;
    }
  }

  // dh0 / dc0, or the fp32 carries of a stack's chunk
#pragma unroll
  for (int s = 0; s < EPTM; ++s) {
    if (own[s] && a.carry_out) {
      a.carry[c_off(s)] = dhc[s];
      a.carry[(int64_t)a.B * a.H + c_off(s)] = dcc[s];
    } else if (own[s]) {
      ((T*)a.dh0)[c_off(s)] = Elem<T>::from_f(dhc[s]);
      ((T*)a.dc0)[c_off(s)] = Elem<T>::from_f(dcc[s]);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int NBT, int MT, int NW, bool DEF>
static hipError_t bwd_col_nkb(const Plan& p, Launch<BwdArgs>& a, hipStream_t s) {
  const int nt = 64 * NW;
  switch (p.bwd_nkb) {
    case 1: return coop_launch(bwd_col_kernel<T, NBT, MT, 1, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
    case 2: return coop_launch(bwd_col_kernel<T, NBT, MT, 2, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
    case 4: return coop_launch(bwd_col_kernel<T, NBT, MT, 4, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
    case 8: return coop_launch(bwd_col_kernel<T, NBT, MT, 8, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
    case 16: return coop_launch(bwd_col_kernel<T, NBT, MT, 16, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
    case 32:
      if constexpr (MT == 1) return coop_launch(bwd_col_kernel<T, NBT, MT, 32, NW, DEF>, launch_grid(p, a), p.lds_bwd, &a, s, nt);
      break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int NW, bool DEF>
static hipError_t bwd_col_nw(const Plan& p, Launch<BwdArgs>& a, hipStream_t s) {
  const int nbt = p.NB < 16 ? 1 : p.NB / 16;
  if (p.bwd_mt == 1) {
    if (nbt == 1) return bwd_col_nkb<T, 1, 1, NW, DEF>(p, a, s);
    if (nbt == 2) return bwd_col_nkb<T, 2, 1, NW, DEF>(p, a, s);
    if (nbt == 4) return bwd_col_nkb<T, 4, 1, NW, DEF>(p, a, s);
  } else if (p.bwd_mt == 2) {
    if (nbt == 1) return bwd_col_nkb<T, 1, 2, NW, DEF>(p, a, s);
    if (nbt == 2) return bwd_col_nkb<T, 2, 2, NW, DEF>(p, a, s);
    if (nbt == 4) return bwd_col_nkb<T, 4, 2, NW, DEF>(p, a, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int NW>
static hipError_t bwd_col_def(const Plan& p, Launch<BwdArgs>& a, hipStream_t s) {
  return p.xcd_local ? bwd_col_nw<T, NW, true>(p, a, s) : bwd_col_nw<T, NW, false>(p, a, s);
}

hipError_t launch_bwd_col(const Plan& p, Launch<BwdArgs>& a, hipStream_t s) {
  if (p.NB * p.NJ > 1024) return hipErrorInvalidValue;
  if (p.dtype == 1) return p.waves == 8 ? bwd_col_def<bf16_t, 8>(p, a, s) : bwd_col_def<bf16_t, kWaves>(p, a, s);
  if (p.dtype == 2) return p.waves == 8 ? bwd_col_def<f16_t, 8>(p, a, s) : bwd_col_def<f16_t, kWaves>(p, a, s);
  if (p.waves != kWaves) return hipErrorInvalidValue;
  return bwd_col_def<float, kWaves>(p, a, s);
}

}  // namespace lstm
