// mfma_probe.hip -- the parts of a stage of the pipelined bf16 products
// (gemm.hip), one at a time, on the whole device: what each costs the
// matrix cores.
//
// A stage of gemm_lds_kernel, per work-group of 8 waves (two per SIMD) and
// 256 x 256 tile: wait for the stage's direct-to-LDS loads, a barrier, four
// direct-to-LDS loads per wave for a later stage (32 KB per work-group), 12
// fragment reads per wave from LDS (12 KB), then 32
// v_mfma_f32_16x16x32_bf16 per wave.  The probe runs iterations of exactly
// that shape with chosen parts left out:
//   reads       fragment reads before the products (the plain order);
//   reads_ahead fragment reads for the next iteration, issued before this
//               iteration's products (their latency off the products' path);
//   barrier     one work-group barrier per iteration;
//   dma         four direct-to-LDS loads per wave per iteration from a
//               64 KB buffer (L2-resident), three iterations in flight.
// The products always run: 32 MFMAs per wave and iteration on operands in
// registers, accumulating into 32 independent tiles.  Fraction of the
// bf16 dense peak = MFMA FLOPs / time / peak.  Nothing here is part of the
// LSTM path; the kernel only measures.
#include "device_common.hpp"
#include "internal.hpp"

namespace lstm {

template <int PARTS>
__global__ void __launch_bounds__(512, 1) mfma_probe_kernel(const uint32_t* src, float* sink, int iters) {
  constexpr bool kReads = (PARTS & kProbeReads) != 0, kAhead = (PARTS & kProbeReadsAhead) != 0;
  constexpr bool kBarrier = (PARTS & kProbeBarrier) != 0, kDma = (PARTS & kProbeDma) != 0;
  // 48 KB of fragments (four rounds of 12 KB) and 32 KB of direct-to-LDS
  // targets (4 KB per wave)
  __shared__ __attribute__((aligned(16))) char lds[80 * 1024];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 48 * 1024 / 4; i += 512)
    ((uint32_t*)lds)[i] = 0x3c003c00u ^ ((uint32_t)(i * 2654435761u) & 0x000f000fu);  // small bf16 values
  __syncthreads();
  u32x4_t a[8], b[4], na[8], nb[4];
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the 12 fragments of round it: 1 KB each, 16 bytes per lane
  auto frags = [&](int it, u32x4_t (&oa)[8], u32x4_t (&ob)[4]) {
    const char* base = lds + (it & 3) * 12 * 1024 + lane * 16;
#pragma unroll
    for (int f = 0; f < 4; ++f) ob[f] = *(const u32x4_t*)(base + f * 1024);
#pragma unroll
    for (int f = 0; f < 8; ++f) oa[f] = *(const u32x4_t*)(base + (4 + f) * 1024);
  };
  frags(0, a, b);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, 64 * 1024, 0x00020000);
  const uint32_t dlds = (uint32_t)(uintptr_t)(lds_void_t*)lds + 48 * 1024 + (uint32_t)w * 4096;
  for (int it = 0; it < iters; ++it) {
    if constexpr (kDma) {
      // four 1 KB loads of this wave (offsets inside the 64 KB buffer), then
      // at most three iterations' loads outstanding
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lds_dma16_at<false>(r, dlds + j * 1024, (uint32_t)(lane * 16 + (((it * 4 + j) & 63) << 10)), 0u);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(12));
    }
    if constexpr (kBarrier) __builtin_amdgcn_s_barrier();
    if constexpr (kReads) {
      frags(it + 1, a, b);
    } else if constexpr (kAhead) {
      frags(it + 1, na, nb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = Mfma<bf16_t>::mac(b[j], a[i], acc[i][j]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kAhead && !kReads) {
#pragma unroll
      for (int f = 0; f < 8; ++f) a[f] = na[f];
#pragma unroll
      for (int f = 0; f < 4; ++f) b[f] = nb[f];
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  sink[(int64_t)blockIdx.x * 512 + tid] = s;
}

template <int PARTS>
static hipError_t probe_parts(int grid, const uint32_t* src, float* sink, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel<PARTS>, dim3((unsigned)grid), dim3(512), 0, s, src, sink, iters);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int parts, int grid, const uint32_t* src, float* sink, int iters, hipStream_t s) {
  constexpr int R = kProbeReads, A = kProbeReadsAhead, B = kProbeBarrier, D = kProbeDma;
  switch (parts) {
    case 0: return probe_parts<0>(grid, src, sink, iters, s);
    case R: return probe_parts<R>(grid, src, sink, iters, s);
    case A: return probe_parts<A>(grid, src, sink, iters, s);
    case B: return probe_parts<B>(grid, src, sink, iters, s);
    case D: return probe_parts<D>(grid, src, sink, iters, s);
    case R | B: return probe_parts<R | B>(grid, src, sink, iters, s);
    case A | B: return probe_parts<A | B>(grid, src, sink, iters, s);
    case R | D: return probe_parts<R | D>(grid, src, sink, iters, s);
    case A | D: return probe_parts<A | D>(grid, src, sink, iters, s);
    case B | D: return probe_parts<B | D>(grid, src, sink, iters, s);
    case R | B | D: return probe_parts<R | B | D>(grid, src, sink, iters, s);
    case A | B | D: return probe_parts<A | B | D>(grid, src, sink, iters, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lstm
