// Matrix-core throughput and clock probe, and an HBM copy probe, for gfx950.
// Measurement only: no step of the attention path runs here. They give the
// benchmark the bf16 MFMA rate the chip actually sustains (and the core clock it
// sustains it at) beside the published dense peak, which assumes 2.4 GHz, and the
// memory bandwidth a plain streaming copy reaches beside the 8 TB/s spec.
//
// Every wave runs four independent accumulation chains of
// v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 multiply-adds, 32768 FLOP each) for
// `iters` iterations on operands held in registers, so nothing but the matrix
// cores is exercised. Wave 0 of each workgroup reads the core-clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) around its loop;
// their ratio is the core clock during the loop. Each workgroup holds 96 KB of
// LDS (otherwise unused), so at most one is resident on a compute unit: a grid
// of one per compute unit puts one wave on every SIMD, all running at once, and
// four independent chains keep that SIMD's matrix core busy (one product per 32
// core cycles). With two waves per SIMD the pair progresses unevenly, which
// blurs the per-workgroup clock reading.
#include "jfa_internal.h"
#include "jfa_device.h"

using namespace jfa_dev;

namespace {

constexpr int kProbeThreads = 256;          // four waves
constexpr int kProbeLdsFloats = 96 * 256;   // 96 KB: one workgroup per compute unit

__global__ void __launch_bounds__(kProbeThreads) mfma_probe_kernel(int iters, float* sink,
                                                                   unsigned long long* clocks) {
  __shared__ float pad[kProbeLdsFloats];
  const uint32_t lane = threadIdx.x & 63;
  // bf16 operands near 2^-7 (0x3C00), varied per lane so no value is special
  const u32x4 a = {0x3C003C00u ^ lane, 0x3C013C02u, 0x3C033C04u ^ lane, 0x3C053C06u};
  const u32x4 b = {0x3C073C08u, 0x3C093C0Au ^ lane, 0x3C0B3C0Cu, 0x3C0D3C0Eu ^ lane};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  // the counters are read once the last products have been consumed
  asm volatile("" ::"v"(s));
  // touch the LDS reservation (a dynamic index keeps all of it allocated)
  pad[(threadIdx.x * 96 + iters) % kProbeLdsFloats] = s;
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  sink[int64_t(blockIdx.x) * kProbeThreads + threadIdx.x] =
      pad[(threadIdx.x * 96 + iters) % kProbeLdsFloats];
  if (threadIdx.x == 0) {
    unsigned long long* c = clocks + 4 * int64_t(blockIdx.x);
    c[0] = t1 - t0;
    c[1] = r1 - r0;
    c[2] = r0;
    c[3] = r1;
  }
}

// Streaming copy for the HBM probe: each thread moves UNROLL 16-byte vectors per
// pass (all loads issued before the stores, so a wave keeps UNROLL loads in
// flight), grid-striding over n16 vectors. Every access is at an index < n16.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ void __launch_bounds__(kCopyThreads) copy_probe_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst,
                                                                  int64_t n16) {
  const int64_t step = int64_t(gridDim.x) * kCopyThreads * kCopyUnroll;
  for (int64_t base = int64_t(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x; base < n16;
       base += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + int64_t(u) * kCopyThreads;
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + int64_t(u) * kCopyThreads;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

}  // namespace

extern "C" jfa_status jfa_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t workgroups,
                                     void* stream) {
  jfa::set_error("");
  if (!src || !dst) return jfa::fail(JFA_ERR_INVALID_ARG, "src and dst must be device pointers");
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16 || bytes % 16)
    return jfa::fail(JFA_ERR_INVALID_ARG, "src, dst and bytes must be multiples of 16");
  if (workgroups < 1 || workgroups > 65536)
    return jfa::fail(JFA_ERR_INVALID_ARG, "workgroups must be in [1, 65536]");
  if (bytes == 0) return JFA_OK;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(workgroups), dim3(kCopyThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), int64_t(bytes / 16));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("copy probe launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

extern "C" jfa_status jfa_probe_mfma(int32_t iters, int32_t workgroups, float* sink,
                                     uint64_t* clocks, void* stream) {
  jfa::set_error("");
  if (iters < 1 || iters > (1 << 24)) return jfa::fail(JFA_ERR_INVALID_ARG, "iters must be in [1, 2^24]");
  if (workgroups < 1 || workgroups > 65536)
    return jfa::fail(JFA_ERR_INVALID_ARG, "workgroups must be in [1, 65536]");
  if (!sink || !clocks) return jfa::fail(JFA_ERR_INVALID_ARG, "sink and clocks must be device pointers");
  if (reinterpret_cast<uintptr_t>(sink) % 4 || reinterpret_cast<uintptr_t>(clocks) % 8)
    return jfa::fail(JFA_ERR_INVALID_ARG, "sink must be 4-byte and clocks 8-byte aligned");
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), int(iters), sink,
                     reinterpret_cast<unsigned long long*>(clocks));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("probe launch: ") + hipGetErrorString(e));
  return JFA_OK;
}
