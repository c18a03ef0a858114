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
// W_h per wave, NBT 16-row batch tiles, C ring chunks in flight per thread
// (0: direct-to-LDS copy), NW waves (8-wave work-groups hold twice the W_h
// slice of 4-wave ones), MW M-tiles per wave.
//
// Waves: the NJ/4 M-tiles (16 interleaved gate rows = 4 units each) form
// groups of MW; the KS = NW*MW/(NJ/4) waves of a group split k, each taking
// all MW M-tiles of the group over its k part, so one LDS read of h feeds MW
// products (the product is bound by LDS reads of h).  Wave wk < MW of a
// group owns M-tile wk of it: it receives the other waves' partial sums of
// that tile and runs its elementwise step.
#include "recurrent_common.hpp"

namespace lstm {

// ---------------------------------------------------------------------------
template <typename T, int NBT, int NKBW, int C, int NW, int MW, bool TG>
__global__ void __launch_bounds__(64 * NW, 1) fwd_rec_kernel(Launch<FwdArgs> L) {
  constexpr int NTH = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int E = sizeof(T);
  constexpr int KB = Mfma<T>::kBlock;
  // the wave index is uniform (branches on it are scalar: an s_waitcnt under
  // a divergent branch would run for every wave)
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15, fq = lane >> 4;
  FwdArgs a;
  const int wgi = slot_select(L, a);
  int bg, jg;
  take_role(wgi, a.nBG, a.nJG, a.nxcd, a.local, a.misplace, bg, jg);
  claim_role(a.claims, bg * a.nJG + jg, a.err);
  const bool local = a.local != 0;
  const int b0 = bg * a.NB, j0 = jg * a.NJ;
  const int MT = a.NJ / 4;                   // M-tiles (16 interleaved gate rows = 4 units)
  const int KS = NW * MW / MT;               // waves splitting k per group of MW M-tiles
  const int mg = w / KS, wk = w % KS;        // this wave's M-tile group and k part
  const bool owner = wk < MW;                // owns M-tile mg*MW + wk
  const int mt = mg * MW + (owner ? wk : 0); // the owned M-tile
  const int kb0 = wk * NKBW;
  const int strideH = a.Hp * E + 16;         // LDS row of h_{t-1}
  const int NBr = a.NB < 16 ? 16 : a.NB;     // rows of the batch tiles (rows >= NB stay zero)
  char* Hl = smem;                           // [NBr][strideH]
  float* red = (float*)(smem + NBr * strideH);  // [MT*(KS-1) partial slots][NBT][64][4]
  const int64_t G4 = 4 * (int64_t)a.H;
  const int u = j0 + 4 * mt + fq;            // unit of this lane's elementwise results
  bool dead = false;

  // --- resident W_h fragments: rows 16*(mg*MW + mi) + fr (gate fr&3 of unit
  // 4*(mg*MW + mi) + fr/4), k-blocks kb0 + i.  Gathered through a
  // wave-private LDS area in passes of PB k-blocks: the wave reads its 16 rows
  // with consecutive lanes on consecutive columns, and every lane then takes
  // each of its fragments with one 16-byte LDS read.
  u32x4_t wreg[MW][NKBW];
#pragma unroll
  for (int mi = 0; mi < MW; ++mi) {
    constexpr int PB = NKBW < 8 ? NKBW : 8;             // k-blocks per pass (8 KB of LDS per wave)
    constexpr int CWL = PB * KB;                        // staged columns per row
    constexpr int RSW = CWL + 16 / E;                   // staged row (elements), padded
    constexpr int LPT = 16 * CWL / 64;                  // elements each lane loads per pass
    T* stage = (T*)smem + w * 16 * RSW;
#pragma unroll
    for (int p = 0; p < NKBW / PB; ++p) {
      T v[LPT];
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int e = lane + 64 * j, row = e / CWL, col = e % CWL;
        const int ur = j0 + 4 * (mg * MW + mi) + (row >> 2), g = row & 3;
        const int k = (kb0 + p * PB) * KB + col;
        const bool ok = ur < a.H && k < a.H;
        v[j] = ((const T*)a.W)[ok ? ((int64_t)gate_block(g, a.ijfo) * a.H + ur) * a.Z + k : 0];
        v[j] = ok ? v[j] : T(0);
      }
#pragma unroll
      for (int j = 0; j < LPT; ++j) {
        const int e = lane + 64 * j;
        stage[(e / CWL) * RSW + e % CWL] = v[j];
      }
#pragma unroll
      for (int ii = 0; ii < PB; ++ii)
        wreg[mi][p * PB + ii] = *(const u32x4_t*)(stage + fr * RSW + ii * KB + fq * (16 / E));
    }
  }
  __syncthreads();  // the staging area is reused below
  const int NBv = (a.B - b0) < a.NB ? (a.B - b0) : a.NB;  // valid rows of this group
  // --- zero the padding of h_{t-1} in LDS once (k >= H, rows past the group or B)
  for (int idx = tid; idx < NBr * a.Hp; idx += NTH) {
    const int bl = idx / a.Hp, k = idx % a.Hp;
    if (k >= a.H || bl >= NBv) *(T*)(Hl + bl * strideH + k * E) = T(0);
  }
  // --- cell state of this lane's elements (owner waves run the elementwise)
  float cst[NBT];
#pragma unroll
  for (int nt = 0; nt < NBT; ++nt) {
    const int b = b0 + 16 * nt + fr;
    const bool ok = u < a.H && 16 * nt + fr < NBv;
    cst[nt] = !ok ? 0.f : a.c0f ? a.c0f[(int64_t)b * a.H + u] : a.c0 ? ldf<T>(a.c0, (int64_t)b * a.H + u) : 0.f;
  }
  // packed h ring: row b of slot s at byte ((s * Bp + b) * Hp) * E; the chunks
  // covering [0, H) of the group's valid rows are read each step
  const int rowB = a.Hp * E;                              // bytes per row
  const int cpr = (a.H * E + 15) / 16;                    // 16-byte chunks per row with data
  const int nchunk = NBv * cpr;
  const __amdgpu_buffer_rsrc_t hd_rsrc = make_rsrc(a.HD, a.hd_bytes);
  T* HDt = (T*)a.HD;

  // Memory traffic off the exchange path (register-copy path): the input
  // projection P_{t+1} and the step's record (y_t, the activated gates, c_t)
  // are issued by the owner lanes right after the ring reads of the next
  // step.  A wave's vector-memory operations complete in issue order, so
  // operations issued before the ring reads would hold up the wait for them;
  // issued after, they drain while the product runs.  Lanes without an
  // element use offsets out of the buffers' range (nothing is moved).
  const int64_t stepP = (int64_t)a.B * G4 * 4;            // bytes of P per step
  const int64_t stepY = (int64_t)a.B * a.H;               // elements of y / Cs per step
  // element (b, u) index in a [B][H] step; lanes without an element address
  // the first byte past each buffer (reads return zeros, writes are dropped)
  int eidx[NBT];
  bool eok[NBT];
#pragma unroll
  for (int nt = 0; nt < NBT; ++nt) {
    const int b = b0 + 16 * nt + fr;
    eok[nt] = u < a.H && 16 * nt + fr < NBv;
    eidx[nt] = b * a.H + u;
  }
  f32x4_t pf[NBT], pfn[NBT];  // P_t (in use) and P_{t+1} (in flight)
  auto load_p = [&](f32x4_t (&dst)[NBT], int tt) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.P + (int64_t)(tt < a.T ? mem_t(tt, a.T, a.rev) : 0) * (stepP / 4)), 0, tt < a.T ? (int)stepP : 0,
        0x00020000);
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt)
      dst[nt] = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, eok[nt] ? 16 * eidx[nt] : (int)stepP, 0, 0));
  };
  T hq[NBT];        // h of this lane's elements: h0, then the state after each step
  float cq[NBT];
  u32x4_t gq[NBT];  // activated gates of the step, packed (E == 2: two words)
  int lenb[NBT];    // sequence length of each element's batch row
#pragma unroll
  for (int nt = 0; nt < NBT; ++nt) {
    hq[nt] = (a.h0 && eok[nt]) ? ((const T*)a.h0)[eidx[nt]] : T(0);
    lenb[nt] = eok[nt] ? len_of(a.len, b0 + 16 * nt + fr, a.T) : a.T;
  }
  auto store_record = [&](int tt) {
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((T*)a.y + mem_t(tt, a.T, a.rev) * stepY), 0, (int)(stepY * E), 0x00020000);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((T*)a.Gs + mem_t(tt, a.T, a.rev) * stepY * 4), 0, (int)(stepY * 4 * E), 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.Cs + mem_t(tt, a.T, a.rev) * stepY), 0, (int)(stepY * 4), 0x00020000);
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt) {
      const int o = eok[nt] ? eidx[nt] : (int)stepY;  // stepY: one past the end
      if constexpr (E == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, hq[nt]), ry, 4 * o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, gq[nt]), rg, 16 * o, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, hq[nt]), ry, 2 * o, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(v2u32_t{gq[nt][0], gq[nt][1]}, rg, 8 * o, 0, 0);
      }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cq[nt]), rc, 4 * o, 0, 0);
    }
  };
  // Direct-to-LDS path: the ring-read phase moves h_{t-1} alone, and every
  // wave waits for its part of it.  After the product, the waves start
  // P_{t+1} into one of two LDS buffers and write the previous step's record
  // (y, activated gates, c) from an LDS staging area as whole 16-byte pieces
  // of its rows; these drain during the k-part reduction and the gate math
  // and are complete at the publish, which waits for every operation of
  // every wave.  (Issued before the product, their LDS writes and staging
  // reads slowed the product's LDS reads: the forward on T=256 B=256 H=1024
  // went from 1204-1211 to 1154-1160 us with them after it.)  The owners
  // read P_t from LDS and stage the step's record there.
  constexpr bool SPLIT = C == 0;
  // Tagged-word exchange (spread layout): h_t of the group travels as 8-byte
  // words of two values and the step (t + 1) in the HX region [2][Bp][HW],
  // stored after the step without a wait or a flag; a reader polls the words
  // of h_{t-1} until each carries tag t (one round of CW words per thread)
  // and copies their values into Hl.  Two slots suffice: a work-group that
  // rewrites a slot at step t + 2 has read every group member's h_{t+1},
  // which each wrote only after reading the slot's h_t.
  static_assert(!TG || (SPLIT && E == 2 && NW == 8 && NBT == 1), "the tagged exchange's instances");
  constexpr bool TAGOK = TG;
  constexpr int CW = 16;
  constexpr bool tagm = TG;
  const int lgHW = 31 - __builtin_clz(a.HW);
  const int HWv = (a.H + 1) / 2;  // words of a row that carry data
  const __amdgpu_buffer_rsrc_t hx_rsrc = make_rsrc(a.HX, (uint32_t)(2 * a.Bp * a.HW * 8));
  const uint32_t hl_lds = (uint32_t)(uintptr_t)(lds_void_t*)smem;  // LDS address of Hl
  const int lgNJ = 31 - __builtin_clz(a.NJ);
  const int nbj = a.NB * a.NJ;                            // 16-byte P chunks (4 gates) per step
  char* Pl = (char*)(red + MT * (KS - 1) * NBT * 256);    // [2][NB][NJ] chunks, chunk c of row bl at c ^ (bl % NJ)
  const int hSr = a.NJ * E + 16, gSr = 4 * a.NJ * E + 16, cSr = 4 * a.NJ + 16;  // padded staging rows (bytes)
  const uint32_t pl_lds = (uint32_t)(uintptr_t)(lds_void_t*)smem + (uint32_t)(Pl - smem);  // LDS address of Pl
  char* hS = Pl + 2 * nbj * 16;                           // [NB][NJ] h
  char* gS = hS + a.NB * hSr;                             // [NB][NJ][4] activated gates
  char* cS = gS + a.NB * gSr;                             // [NB][NJ] c (fp32)
  // Per-lane pieces of these copies, fixed for the launch: wave-load j = w +
  // NW*i of P moves chunk slot 64j + lane; record piece i of a tensor is
  // piece tid + NTH*i of its NBv rows (16 bytes each), at an LDS source and a
  // byte offset in the step's slab of the tensor (out of range when the
  // piece does not exist: the store is dropped)
  constexpr int RJ = (NBT * 8 + NW - 1) / NW;             // P wave-loads per wave, at most
  constexpr int RY = (NBT * 64 * E + NTH - 1) / NTH;      // y pieces per lane (NB <= 16*NBT, NJ <= 32)
  constexpr int RG = (NBT * 256 * E + NTH - 1) / NTH;     // gate pieces
  constexpr int RC = (NBT * 128 + NTH - 1) / NTH;         // c pieces
  uint32_t pvo[RJ], yso[RY], yvo[RY], gso[RG], gvo[RG], cso[RC], cvo[RC];
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < RJ; ++i) {
      const int sl = 64 * (w + NW * i) + lane, bl = sl >> lgNJ;
      const int c = (sl & (a.NJ - 1)) ^ (bl & (a.NJ - 1));
      pvo[i] = (uint32_t)(((b0 + bl) * G4 + 4 * (j0 + c)) * 4);
    }
    const int hC = a.NJ * E / 16, gC = 4 * a.NJ * E / 16, cC = a.NJ / 4;
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_void_t*)smem;
#pragma unroll
    for (int i = 0; i < RY; ++i) {
      const int q = tid + NTH * i, bl = q / hC, c = q - bl * hC;
      const bool ok = q < NBv * hC;
      yso[i] = ok ? smem_lds + (uint32_t)(hS - smem) + bl * hSr + 16 * c : smem_lds;
      yvo[i] = ok ? (uint32_t)(((b0 + bl) * a.H + j0) * E + 16 * c) : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int q = tid + NTH * i, bl = q / gC, c = q - bl * gC;
      const bool ok = q < NBv * gC;
      gso[i] = ok ? smem_lds + (uint32_t)(gS - smem) + bl * gSr + 16 * c : smem_lds;
      gvo[i] = ok ? (uint32_t)(((b0 + bl) * G4 + 4 * j0) * E + 16 * c) : 0x80000000u;
    }
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int q = tid + NTH * i, bl = q / cC, c = q - bl * cC;
      const bool ok = q < NBv * cC;
      cso[i] = ok ? smem_lds + (uint32_t)(cS - smem) + bl * cSr + 16 * c : smem_lds;
      cvo[i] = ok ? (uint32_t)(((b0 + bl) * a.H + j0) * 4 + 16 * c) : 0x80000000u;
    }
  }
  auto dma_p = [&](int tt) {
    // P_tt of the group's rows and units into buffer tt & 1; rows past B are
    // out of the buffer's range (zeros)
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.P + (int64_t)mem_t(tt, a.T, a.rev) * (stepP / 4)), 0, (int)stepP, 0x00020000);
    const uint32_t dst = pl_lds + (uint32_t)((tt & 1) * nbj * 16);
#pragma unroll
    for (int i = 0; i < RJ; ++i) {
      const int j = w + NW * i;
      if (64 * j < nbj && 64 * j + lane < nbj) lds_dma16_at<false>(r, dst + 64 * j * 16, pvo[i], 0u);
    }
  };
  auto store_rec = [&](int tt) {
    // the record of step tt from the staging area: every piece read, then
    // every piece stored
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((T*)a.y + mem_t(tt, a.T, a.rev) * stepY), 0, (int)(stepY * E), 0x00020000);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((T*)a.Gs + mem_t(tt, a.T, a.rev) * stepY * 4), 0, (int)(stepY * 4 * E), 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.Cs + mem_t(tt, a.T, a.rev) * stepY), 0, (int)(stepY * 4), 0x00020000);
    typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
    u32x4_t vy[RY], vg[RG], vc[RC];
#pragma unroll
    for (int i = 0; i < RY; ++i) vy[i] = *(lds_u4*)(uintptr_t)yso[i];
#pragma unroll
    for (int i = 0; i < RG; ++i) vg[i] = *(lds_u4*)(uintptr_t)gso[i];
#pragma unroll
    for (int i = 0; i < RC; ++i) vc[i] = *(lds_u4*)(uintptr_t)cso[i];
#pragma unroll
    for (int i = 0; i < RY; ++i) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, vy[i]), ry, yvo[i], 0, 0);
#pragma unroll
    for (int i = 0; i < RG; ++i) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, vg[i]), rg, gvo[i], 0, 0);
#pragma unroll
    for (int i = 0; i < RC; ++i) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, vc[i]), rc, cvo[i], 0, 0);
  };
  if (SPLIT) {
    dma_p(0);
    wait_vmem();
    __syncthreads();
  } else if (owner) {
    load_p(pf, 0);
  }

  for (int t = 0; t < a.T; ++t) {
    stamp(a.stamps, a.T, t, 0);
    inject_failure(a.fail_step, t, wgi, a.err, dead);
    // wait until every work-group of the batch group has published h_{t-1}
    if (t > 0 && !tagm && tid < a.nJG) wait_flag(a.HF + bg * a.nJG + tid, (uint32_t)t, a.err, dead);
    __syncthreads();  // flags seen; the previous step's readers of Hl are done
    stamp(a.stamps, a.T, t, 1);
    // h_{t-1} -> LDS, then the deferred operations
    if (t == 0) {
      for (int idx = tid; idx < NBv * a.H; idx += NTH) {
        const int bl = idx / a.H, k = idx % a.H;
        const T v = a.h0 ? ((const T*)a.h0)[(int64_t)(b0 + bl) * a.H + k] : T(0);
        *(T*)(Hl + bl * strideH + k * E) = v;
      }
      if (!SPLIT && owner) load_p(pfn, 1);
      wait_vmem();
      __syncthreads();
    } else {
      const uint32_t slot0 = (uint32_t)(((t - 1) & 1) * a.Bp + b0) * (uint32_t)rowB;
      if constexpr (C == 0) {
        bool tagged = false;
        if constexpr (TAGOK) {
          if (tagm) {
            // word q = bl * HW + w of the group's rows in slot (t - 1) & 1,
            // q = tid + NTH * c; 8-byte device-coherent loads, re-polled
            // until each carries tag t (bounded as every other wait)
            // P_{t+1} and the previous step's record first: they drain
            // while the words of the other work-groups arrive (issued after
            // the product's start, they would also hold up any wait for a
            // spilled operand there)
            if (t + 1 < a.T) dma_p(t + 1);
            store_rec(t - 1);
            const uint32_t sbase = (uint32_t)((((t - 1) & 1) * a.Bp + b0) * a.HW) * 8u;
            const int nq = NBv << lgHW;
            uint64_t wv[CW];
            uint32_t pend = 0;
#pragma unroll
            for (int c = 0; c < CW; ++c) {
              const int q = tid + NTH * c;
              const bool ok = q < nq && (q & (a.HW - 1)) < HWv;
              pend |= (ok ? 1u : 0u) << c;
              wv[c] = ok ? __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(hx_rsrc, 8 * q, sbase, 16))
                         : 0ull;
            }
            if (!dead) {
              uint64_t w0 = 0;
              uint32_t rounds = 0;
              while (true) {
                uint32_t miss = 0;
#pragma unroll
                for (int c = 0; c < CW; ++c)
                  if (((pend >> c) & 1u) && (uint32_t)(wv[c] >> 32) != (uint32_t)t) miss |= 1u << c;
                if (!miss) break;
                if (w0 == 0) {
                  w0 = now_ticks();
                } else if ((++rounds & 15u) == 0 && (now_ticks() - w0 > kWaitTicks || err_set(a.err))) {
                  atomicOr(a.err, kErrTimeout);
                  dead = true;
                  break;
                }
#pragma unroll
                for (int c = 0; c < CW; ++c)
                  if ((miss >> c) & 1u)
                    wv[c] = __builtin_bit_cast(
                        uint64_t, __builtin_amdgcn_raw_buffer_load_b64(hx_rsrc, 8 * (tid + NTH * c), sbase, 16));
              }
            }
            wait_vmem();
#pragma unroll
            for (int c = 0; c < CW; ++c)
              if ((pend >> c) & 1u) {
                const int q = tid + NTH * c, bl = q >> lgHW, wd = q & (a.HW - 1);
                *(uint32_t*)(Hl + bl * strideH + wd * 4) = (uint32_t)wv[c];
              }
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            tagged = true;
          }
        }
        if (!tagged) {
          // direct-to-LDS: wave-load j moves chunks [64j, 64j + 64) -- 1 KB
          // of one row, as every row holds a multiple of 64 chunks here
          // (device-coherent loads, issued as inline asm and waited for
          // explicitly: the compiler's own waits for the builtin form
          // measured slower where the ring is read across XCDs)
          for (int j = w; j * 64 < nchunk; j += NW) {
            const int bl = (64 * j) / cpr, cc = 64 * j - bl * cpr;
            lds_dma16_at<true>(hd_rsrc, hl_lds + (uint32_t)(bl * strideH + cc * 16),
                               slot0 + (uint32_t)(bl * rowB + lane * 16), (uint32_t)(cc * 16));
          }
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
      } else {
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
      if constexpr (!SPLIT) {
        asm volatile("" ::: "memory");
        if (owner) {
          store_record(t - 1);
          load_p(pfn, t + 1);
        }
        asm volatile("" ::: "memory");
        // register path: the ring's LDS writes are done once lgkmcnt is 0
        __builtin_amdgcn_s_waitcnt(kLgkm0);
      }
      // the barrier then covers the other waves
      __builtin_amdgcn_s_barrier();
    }
    stamp(a.stamps, a.T, t, 2);

    // MFMA: part[mi][nt] = W_h[rows of M-tile mg*MW + mi, k part] .
    // h_{t-1}[tile nt]^T, with CH independent accumulator chains per tile
    // (summed in a fixed order); one LDS read of h feeds the MW tiles
    constexpr int CH = NBT * MW == 1 ? (NKBW >= 4 ? 4 : NKBW) : (NBT * MW == 2 && NKBW >= 2 ? 2 : 1);
    f32x4_t acc[MW][NBT], part[MW][NBT][CH];
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt)
#pragma unroll
        for (int ch = 0; ch < CH; ++ch) part[mi][nt][ch] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The B fragments are read in chunks of CKF k-blocks into two register
    // buffers, the next chunk's reads issued ahead of the current chunk's
    // products (scheduling barriers keep the compiler from trading the reads
    // in flight for registers and waiting on every read).  A pass covers
    // batch tiles [NT0, NT0 + NTN); one pass covers them all.
    const char* hb0 = Hl + fr * strideH + kb0 * 64 + fq * 16;
    auto product = [&](auto nt0c, auto ntnc) {
      constexpr int NT0 = decltype(nt0c)::value, NTN = decltype(ntnc)::value;
      constexpr int CKF0 = 4 / NTN > 0 ? 4 / NTN : 1;
      constexpr int CKF = NKBW < CKF0 ? NKBW : CKF0;
      constexpr int NCF = NKBW / CKF;
      static_assert(NKBW % CKF == 0, "chunks divide the k-blocks");
      u32x4_t hbuf[2][CKF][NTN];
      auto read_chunk = [&](int cf, int buf) {
#pragma unroll
        for (int ii = 0; ii < CKF; ++ii)
#pragma unroll
          for (int n = 0; n < NTN; ++n)
            hbuf[buf][ii][n] = *(const u32x4_t*)(hb0 + 16 * (NT0 + n) * strideH + (cf * CKF + ii) * 64);
      };
      read_chunk(0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cf = 0; cf < NCF; ++cf) {
        if (cf + 1 < NCF) read_chunk(cf + 1, (cf + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ii = 0; ii < CKF; ++ii) {
          const int i = cf * CKF + ii;
#pragma unroll
          for (int n = 0; n < NTN; ++n)
#pragma unroll
            for (int mi = 0; mi < MW; ++mi)
              part[mi][NT0 + n][i % CH] = Mfma<T>::mac(wreg[mi][i], hbuf[cf & 1][ii][n], part[mi][NT0 + n][i % CH]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    product(std::integral_constant<int, 0>{}, std::integral_constant<int, NBT>{});
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        acc[mi][nt] = part[mi][nt][0];
#pragma unroll
        for (int ch = 1; ch < CH; ++ch) acc[mi][nt] += part[mi][nt][ch];
      }
    stamp(a.stamps, a.T, t, 3);
    // P_{t+1} and the record of step t - 1 (their staging reads come before
    // the barrier below, the staging writes of this step after it)
    if constexpr (SPLIT) {
      if (!tagm || t == 0) {  // (the tagged exchange issues them before its ring read)
        if (t + 1 < a.T) dma_p(t + 1);
        if (t > 0) store_rec(t - 1);
      }
    }
    // k-part reduction: partial tiles go to their owners through LDS; slot
    // (M-tile m, kk) holds the part of the kk-th non-owner wave of m's group
    f32x4_t mine[NBT];
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt) mine[nt] = acc[0][nt];
#pragma unroll
    for (int mi = 1; mi < MW; ++mi)
      if (wk == mi)
#pragma unroll
        for (int nt = 0; nt < NBT; ++nt) mine[nt] = acc[mi][nt];
    if (KS > 1) {
#pragma unroll
      for (int mi = 0; mi < MW; ++mi) {
        if (wk == mi) continue;
        const int m = mg * MW + mi, kk = wk < mi ? wk : wk - 1;
#pragma unroll
        for (int nt = 0; nt < NBT; ++nt)
          *(f32x4_t*)(red + (((m * (KS - 1) + kk) * NBT + nt) * 64 + lane) * 4) = acc[mi][nt];
      }
      // LDS writes done, then the barrier (not __syncthreads: that would
      // also wait for the deferred memory operations)
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
      if (owner) {
        for (int kk = 0; kk < KS - 1; ++kk) {
#pragma unroll
          for (int nt = 0; nt < NBT; ++nt)
            mine[nt] += *(const f32x4_t*)(red + (((mt * (KS - 1) + kk) * NBT + nt) * 64 + lane) * 4);
        }
      }
    }
    // without a k-part reduction no barrier separates the record's staging
    // reads above from the staging writes below
    if (SPLIT && KS == 1) {
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
    }
    stamp(a.stamps, a.T, t, 4);
    // elementwise: gates, cell, hidden; h_t is published (stores, their
    // completion, then the flag), the record is kept for the next step
    if (owner) {
      T* dst = HDt + (int64_t)(t & 1) * a.Bp * a.Hp;
#pragma unroll
      for (int nt = 0; nt < NBT; ++nt) {
        const int b = b0 + 16 * nt + fr;
        const bool valid = u < a.H && 16 * nt + fr < NBv;
        f32x4_t pv;
        if constexpr (SPLIT) {
          const int bl = 16 * nt + fr, ul = u - j0;
          pv = bl < a.NB ? *(const f32x4_t*)(Pl + (t & 1) * nbj * 16 + ((bl << lgNJ) + (ul ^ (bl & (a.NJ - 1)))) * 16)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
        } else {
          pv = pf[nt];
        }
        const f32x4_t z = mine[nt] + pv;
        const float ig = sigmoidf(z[0]), fg = sigmoidf(z[1]), gg = tanh_f(z[2]), og = sigmoidf(z[3]);
        float c = fg * cst[nt] + ig * gg;
        float h = og * tanh_f(c);
        if (mem_t(t, a.T, a.rev) >= lenb[nt]) {  // past the sequence's end: the state is held
          c = cst[nt];
          h = Elem<T>::to_f(hq[nt]);
        }
        cst[nt] = c;
        cq[nt] = c;
        hq[nt] = Elem<T>::from_f(h);
        T g4[4] = {Elem<T>::from_f(ig), Elem<T>::from_f(fg), Elem<T>::from_f(gg), Elem<T>::from_f(og)};
        if constexpr (E == 4) {
          gq[nt] = __builtin_bit_cast(u32x4_t, g4);
        } else {
          const uint64_t g64 = __builtin_bit_cast(uint64_t, g4);
          gq[nt] = u32x4_t{(uint32_t)g64, (uint32_t)(g64 >> 32), 0u, 0u};
        }
        if (valid && !tagm) store_elem<T>(dst + (int64_t)b * a.Hp + u, hq[nt], local);
        if constexpr (SPLIT) {
          const int bl = 16 * nt + fr, ul = u - j0;
          if (bl < a.NB) {
            *(T*)(hS + bl * hSr + ul * E) = hq[nt];
            if constexpr (E == 4)
              *(u32x4_t*)(gS + bl * gSr + ul * 16) = gq[nt];
            else
              *(uint64_t*)(gS + bl * gSr + ul * 8) = (uint64_t)gq[nt][0] | ((uint64_t)gq[nt][1] << 32);
            *(float*)(cS + bl * cSr + ul * 4) = c;
          }
        } else {
          pf[nt] = pfn[nt];
        }
      }
    }
    wait_vmem();
    __syncthreads();
    if (tagm) {
      if constexpr (TAGOK) {
        // h_t of this work-group's units from the staging area: word i of
        // row bl holds units j0 + 2i and j0 + 2i + 1 (0 past H)
        const int npair = a.NJ / 2, lgp = 31 - __builtin_clz(npair);
        uint64_t* slot = a.HX + ((int64_t)(t & 1) * a.Bp + b0) * a.HW + (j0 >> 1);
        for (int q = tid; q < NBv * npair; q += NTH) {
          const int bl = q >> lgp, i = q & (npair - 1), u0 = j0 + 2 * i;
          if (u0 < a.H) {
            const uint16_t v0 = *(const uint16_t*)(hS + bl * hSr + 2 * i * E);
            const uint16_t v1 = u0 + 1 < a.H ? *(const uint16_t*)(hS + bl * hSr + (2 * i + 1) * E) : (uint16_t)0;
            xstore_word(slot + (int64_t)bl * a.HW + i,
                        ((uint64_t)(uint32_t)(t + 1) << 32) | ((uint64_t)v1 << 16) | (uint64_t)v0, false);
          }
        }
      }
    } else if (tid == 0) {
      store_flag(a.HF + bg * a.nJG + jg, (uint32_t)(t + 1), local);
    }
    stamp(a.stamps, a.T, t, 5);
  }
  // the last step's record and the final states
  if (SPLIT) {
    store_rec(a.T - 1);
  } else if (owner) {
    store_record(a.T - 1);
  }
  if (owner) {
#pragma unroll
    for (int nt = 0; nt < NBT; ++nt) {
      const int b = b0 + 16 * nt + fr;
      if (u < a.H && 16 * nt + fr < NBv) {
        ((T*)a.hT)[(int64_t)b * a.H + u] = hq[nt];
        ((T*)a.cT)[(int64_t)b * a.H + u] = Elem<T>::from_f(cq[nt]);
      }
    }
  }
  // T == 0 is handled on the host
}

// ---------------------------------------------------------------------------
template <typename T, int NBT, int C, int NW, int MW, bool TG>
static hipError_t fwd_dispatch_mw(const Plan& p, Launch<FwdArgs>& a, hipStream_t s) {
  const int nt = 64 * NW;
  switch (p.fwd_nkbw) {
    case 1: return coop_launch(fwd_rec_kernel<T, NBT, 1, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
    case 2: return coop_launch(fwd_rec_kernel<T, NBT, 2, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
    case 4: return coop_launch(fwd_rec_kernel<T, NBT, 4, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
    case 8: return coop_launch(fwd_rec_kernel<T, NBT, 8, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
    case 16: return coop_launch(fwd_rec_kernel<T, NBT, 16, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
    case 32:
      if constexpr (MW == 1)
        return coop_launch(fwd_rec_kernel<T, NBT, 32, C, NW, MW, TG>, launch_grid(p, a), p.lds_fwd, &a, s, nt);
      break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int NBT, int C, int NW, bool TG = false>
static hipError_t fwd_dispatch_c(const Plan& p, Launch<FwdArgs>& a, hipStream_t s) {
  if (p.fwd_mw == 2) return fwd_dispatch_mw<T, NBT, C, NW, 2, TG>(p, a, s);
  if (p.fwd_mw == 1) return fwd_dispatch_mw<T, NBT, C, NW, 1, TG>(p, a, s);
  return hipErrorInvalidValue;
}

// The ring is copied into LDS by direct-to-LDS loads when every row holds a
// multiple of 64 16-byte chunks (H * E a multiple of 1 KB), else through
// registers, 4 chunks in flight per thread and round.  8-wave work-groups
// have 16-bit storage only.
template <typename T, int NBT>
static hipError_t fwd_dispatch(const Plan& p, Launch<FwdArgs>& a, hipStream_t s) {
  const bool dma = p.fwd_dma != 0;
  if constexpr (sizeof(T) == 2 && NBT == 1)
    if (p.fwd_tag && dma && p.waves == 8) return fwd_dispatch_c<T, NBT, 0, 8, true>(p, a, s);
  if (p.fwd_tag) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 2)
    if (p.waves == 8) return dma ? fwd_dispatch_c<T, NBT, 0, 8>(p, a, s) : fwd_dispatch_c<T, NBT, 4, 8>(p, a, s);
  if (p.waves != kWaves) return hipErrorInvalidValue;
  return dma ? fwd_dispatch_c<T, NBT, 0, kWaves>(p, a, s) : fwd_dispatch_c<T, NBT, 4, kWaves>(p, a, s);
}

hipError_t launch_fwd_recurrent(const Plan& p, const FwdSlot* slots, int nslots, uint32_t* err, uint64_t* stamps,
                                const int32_t* len, hipStream_t s) {
  if (nslots < 1 || nslots > kMaxSlots) return hipErrorInvalidValue;
  Launch<FwdArgs> a{};
  for (int k = 0; k < kMaxSlots; ++k) {
    const FwdSlot& q = slots[k < nslots ? k : 0];
    char* hd = (char*)q.HX;  // the packed ring and its flags share the tagged-word region
    a.s[k] = FwdArgs{q.P, q.W, q.h0, q.c0, q.y, q.hT, q.cT, q.Gs, q.Cs, q.HX, hd,
                     (uint32_t*)(hd + p.off_hflags), (uint32_t)p.off_hflags, err, k == 0 ? stamps : nullptr, q.T,
                     (int)p.B, (int)p.H, (int)q.Z, p.NB, p.NJ, p.nJG, p.Hp, p.Bp,
                     p.esize == 2 ? (p.Hp / 2) : p.Hp, p.nBG, p.nxcd, p.xcd_local, q.rev, p.ijfo,
                     (uint32_t*)(hd + p.off_hclaim), p.fail_step, p.misplace, len, q.c0f};
  }
  a.nslots = nslots;
  a.grid1 = p.grid;
  if (fwd_vec_ok(p)) return launch_fwd_vec(p, a, s);
  const int nbt = p.NB < 16 ? 1 : p.NB / 16;
  if (p.dtype == 1) {
    if (nbt == 1) return fwd_dispatch<bf16_t, 1>(p, a, s);
    if (nbt == 2) return fwd_dispatch<bf16_t, 2>(p, a, s);
    if (nbt == 4) return fwd_dispatch<bf16_t, 4>(p, a, s);
  } else if (p.dtype == 2) {
    if (nbt == 1) return fwd_dispatch<f16_t, 1>(p, a, s);
    if (nbt == 2) return fwd_dispatch<f16_t, 2>(p, a, s);
    if (nbt == 4) return fwd_dispatch<f16_t, 4>(p, a, s);
  } else {
    if (nbt == 1) return fwd_dispatch<float, 1>(p, a, s);
    if (nbt == 2) return fwd_dispatch<float, 2>(p, a, s);
    if (nbt == 4) return fwd_dispatch<float, 4>(p, a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_recurrent(const Plan& p, const BwdSlot* slots, int nslots, uint32_t* err, uint64_t* stamps,
                                const int32_t* len, hipStream_t s) {
  if (nslots < 1 || nslots > kMaxSlots) return hipErrorInvalidValue;
  Launch<BwdArgs> a{};
  for (int k = 0; k < kMaxSlots; ++k) {
    const BwdSlot& q = slots[k < nslots ? k : 0];
    char* gd = (char*)q.PX;  // the gate-delta ring and its flags share the tagged-word region
    a.s[k] = BwdArgs{q.W, q.c0, q.dy, q.dhT, q.dcT, q.Gs, q.Cs, q.dG, q.PX, gd,
                     (uint32_t*)(gd + p.off_pflags), (uint32_t)p.off_pflags, q.DBP, q.dh0, q.dc0, err,
                     k == 0 ? stamps : nullptr, q.T, (int)p.B, (int)p.H, (int)q.Z, p.NB, p.NJ, p.nJG, p.Hp, p.Bp,
                     p.nBG, p.nxcd, p.xcd_local, q.rev, p.ijfo, (uint32_t*)(gd + p.off_pclaim), p.fail_step,
                     p.misplace, len, q.cprevf, q.carry, q.carry_in, q.carry_out};
  }
  a.nslots = nslots;
  a.grid1 = p.grid;
  if (p.bwd_valu) return launch_bwd_vec(p, a, s);
  return launch_bwd_col(p, a, s);
}

}  // namespace lstm
